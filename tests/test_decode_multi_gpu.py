"""pa_decode_multi on the GPU: q_per_seq new tokens per sequence scored in one
pass (speculative verification), each row attending causally to the cache.
Checked against the float64 oracle's causal attention (the rows are the last
q_per_seq positions of each sequence, as in prefill with a cached prefix),
over every supported (heads per kv head, rows per sequence) combination --
including row counts that are not a power of two, which leave padding rows
in the kernel -- and against pa_decode (q_per_seq = 1, bit for bit) and
pa_prefill (same rows)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from paged_harness import bf16_out_to_f64, compare, oracle_pools, place

pytestmark = pytest.mark.gpu


def run_multi(dev, ql):
    case = dev.case
    pa.store_kv(dev.step_k, dev.step_v, dev.step_slots, dev.k_cache, dev.v_cache)
    out = torch.full((case.batch * ql, case.num_q_heads, case.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_decode_multi_workspace(case.batch, ql, case.num_q_heads, case.num_kv_heads)
    pa.decode_multi(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens, ql,
                    case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    return out


def check(case, ql):
    print(f"[decode_multi] {case.name} B={case.batch} Hq={case.num_q_heads} "
          f"Hkv={case.num_kv_heads} q_per_seq={ql} ctx={case.context_lens.tolist()[:8]}", flush=True)
    assert np.all(case.q_lens == ql)
    dev = place(case)
    out = bf16_out_to_f64(run_multi(dev, ql))
    kp, vp = oracle_pools(case)
    q = wl.bits_to_numpy(case.q_all())
    ref = np.concatenate([
        oracle.prefill_seq(q[b * ql:(b + 1) * ql], kp, vp, case.block_table[b],
                           int(case.context_lens[b]), case.scale) for b in range(case.batch)])
    return compare(out, ref, case.name), dev, out


def test_multi_query_decode_workload():
    """64 sequences x 4 new tokens over U{512..4096} cached tokens."""
    check(wl.multi_query_decode(), 4)


# rows per (sequence, kv head) = hq / hkv * ql: up to 4 (and 8 of one token)
# on the vector-ALU kernel, 5..16 of several tokens on the 16-row and 17..32
# on the 32-row matrix-core kernel
@pytest.mark.parametrize("hq,hkv,ql", [(8, 8, 8), (8, 8, 3), (8, 8, 1), (16, 8, 4), (16, 8, 3),
                                       (16, 8, 2), (32, 8, 2), (64, 8, 1), (4, 1, 2),
                                       (16, 8, 5), (16, 8, 6), (32, 8, 5), (32, 8, 6), (32, 8, 3),
                                       (32, 8, 8), (64, 8, 4), (64, 8, 2), (8, 8, 9), (8, 8, 32),
                                       (4, 1, 8)])
def test_decode_multi_group_and_row_counts(hq, hkv, ql):
    ctx = [ql, ql + 1, 63, 64, 65, 255, 257, 700, 1500]
    case = wl.make_case(f"multi_{hq}_{hkv}_{ql}", "prefill", 60 + hq + ql, ctx, hq, hkv,
                        q_lens=[ql] * len(ctx))
    check(case, ql)


def test_decode_multi_one_row_is_pa_decode():
    """q_per_seq = 1 runs the same kernel as pa_decode: identical bits."""
    case = wl.make_case("multi_vs_decode", "prefill", 70, [1, 100, 256, 257, 3000], 32, 8,
                        q_lens=[1] * 5)
    dev = place(case)
    multi = run_multi(dev, 1)
    out = torch.empty_like(multi)
    ws = pa.alloc_decode_workspace(case.batch, 32, 8)
    pa.decode(out, dev.q, dev.k_cache, dev.v_cache, dev.block_table, dev.context_lens,
              case.max_context_len, case.scale, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), multi.view(torch.int16))


def test_decode_multi_matches_prefill():
    case = wl.multi_query_decode()
    dev = place(case)
    multi = bf16_out_to_f64(run_multi(dev, 4))
    out = torch.empty((case.total_q_rows, 16, 128), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_prefill_workspace(case.batch, case.total_q_rows, case.max_q_len, 16, 8,
                                    case.max_blocks_per_seq)
    pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, case.max_q_len, dev.k_cache, dev.v_cache,
               dev.block_table, case.scale, ws)
    torch.cuda.synchronize()
    assert np.abs(bf16_out_to_f64(out) - multi).max() <= 2 * 1.5e-2


def test_speculative_verification_workload():
    """64 sequences each verify 5 drafted tokens plus the next one (6 rows)
    over U{512..4096} cached tokens: 12 rows per (sequence, kv head), the
    16-row matrix-core kernel."""
    check(wl.spec_verify_decode(), 6)


def test_speculative_verification_four_heads_per_kv_head():
    """The same batch at 32 q / 8 kv heads: 24 rows per (sequence, kv head),
    the 32-row matrix-core kernel, at the size the benchmark times."""
    check(wl.spec_verify_decode_g4(), 6)


@pytest.mark.parametrize("hq", [16, 32])
def test_decode_multi_many_rows_matches_prefill(hq):
    """The same rows through pa_prefill (a varlen batch with q_len = 6 and a
    cached prefix): both within the oracle bar and close to each other."""
    lens = [6, 7, 100, 300, 1000, 2000, 4097]
    case = wl.make_case(f"multi_vs_prefill_{hq}", "prefill", 80 + hq, lens, hq, 8, q_lens=[6] * len(lens))
    _, dev, multi = check(case, 6)
    out = torch.empty((case.total_q_rows, hq, 128), dtype=torch.bfloat16, device="cuda")
    ws = pa.alloc_prefill_workspace(case.batch, case.total_q_rows, case.max_q_len, hq, 8,
                                    case.max_blocks_per_seq)
    pa.prefill(out, dev.q, dev.cu_q, dev.context_lens, case.max_q_len, dev.k_cache, dev.v_cache,
               dev.block_table, case.scale, ws)
    torch.cuda.synchronize()
    pre = bf16_out_to_f64(out)
    assert np.abs(multi - pre).max() <= 1.5e-2


@pytest.mark.parametrize("hq", [16, 32])
def test_decode_multi_long_contexts_cut_across_waves(hq):
    """Few long sequences with 6 rows at 16 or 32 q / 8 kv heads (12 or 24
    rows per kv head: the 16-row and the 32-row matrix-core kernel): every
    segment is cut into many runs and merged from partial records."""
    case = wl.make_case(f"multi_long_{hq}", "prefill", 88, [40000, 70001, 6, 9000], hq, 8, q_lens=[6] * 4)
    check(case, 6)


@pytest.mark.parametrize("hq,ql", [(16, 2), (16, 6), (32, 6)])
def test_decode_multi_block_permutation_gives_identical_bits(hq, ql):
    """Same logical contents under another physical placement, on each of
    the three decode-multi kernels (4, 12 and 24 rows per kv head): the
    split plan depends only on the lengths, so the bits are identical."""
    lens = [ql, 700, 3000, 257, 9000]
    c1 = wl.make_case(f"perm_m{hq}_{ql}", "prefill", 91, lens, hq, 8, q_lens=[ql] * 5, num_blocks=60)
    c2 = wl.make_case(f"perm_m{hq}_{ql}", "prefill", 91, lens, hq, 8, q_lens=[ql] * 5, num_blocks=60,
                      rng=np.random.default_rng(997))
    assert not np.array_equal(c1.block_table, c2.block_table)
    o1 = run_multi(place(c1), ql)
    o2 = run_multi(place(c2), ql)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_decode_multi_negative_scale():
    """A negative logit scale (allowed: finite) on the three decode-multi
    kernels (4, 12 and 24 rows per kv head)."""
    for hq, ql in ((16, 2), (16, 6), (32, 6)):
        case = wl.make_case(f"multi_negscale_{hq}", "prefill", 90 + hq, [ql, 70, 700, 3000], hq, 8,
                            q_lens=[ql] * 4, scale=-0.09)
        check(case, ql)
