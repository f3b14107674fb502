"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-worked layout offsets and closed forms (tests/golden/), a library routine
(torch's float64 scaled-dot-product attention) on contiguous caches, algebraic
invariants, and pure-Python brute force on tiny shapes."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
POISON = wl.POISON_BF16


def f2bf(x) -> np.ndarray:
    """float -> bf16 bits by truncation; only used on values exact in bf16."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def rand_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32).view(np.uint32)
    return ((x.astype(np.uint64) + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)


def build_pools(case: wl.PagedCase, k_rows: np.ndarray, v_rows: np.ndarray, fill=POISON):
    kp, vp = oracle.new_pools(case.num_blocks, case.num_kv_heads, case.head_dim,
                              case.block_size, fill)
    oracle.store_kv(kp, vp, k_rows, v_rows, case.slot_mapping_all)
    return kp, vp


def small_case(seed, lens, hq, hkv, d=16, bs=4, kind="decode", q_lens=None, extra_blocks=3,
               q_mult=1.0):
    used = sum(wl.blocks_for(n, bs) for n in lens)
    return wl.make_case(f"small{seed}", kind, seed, lens, hq, hkv, q_lens=q_lens,
                        num_blocks=used + extra_blocks, head_dim=d, block_size=bs, q_mult=q_mult)


def case_tensors(case):
    k = wl.bits_to_numpy(case.k_rows(0, case.total_kv_rows))
    v = wl.bits_to_numpy(case.v_rows(0, case.total_kv_rows))
    q = wl.bits_to_numpy(case.q_all())
    return q, k, v


def sdpa(q, k, v, scale, causal=False):
    """torch float64 SDPA; q [Hq, R, D], k/v [Hq, n, D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=causal, scale=scale)[0].numpy()


# ---------------------------------------------------------------- layout / store

def test_layout_offsets_match_hand_worked_values():
    g = json.load(open(os.path.join(GOLDEN, "layout_offsets.json")))
    hkv, d, bs = g["num_kv_heads"], g["head_dim"], g["block_size"]
    nb = 1 + max(c["slot"] for c in g["cases"]) // bs
    for c in g["cases"]:
        kp, vp = oracle.new_pools(nb, hkv, d, bs, 0)
        # marker values: distinct per (head, dim), never 0
        k_new = (np.arange(hkv * d, dtype=np.uint16) + 1).reshape(1, hkv, d)
        v_new = k_new + np.uint16(20000)
        oracle.store_kv(kp, vp, k_new, v_new, np.array([c["slot"]], np.int32))
        assert kp.reshape(-1)[c["k_offset"]] == k_new[0, c["head"], c["d"]], c
        assert vp.reshape(-1)[c["v_offset"]] == v_new[0, c["head"], c["d"]], c
        # exactly one token's worth of elements was written
        assert np.count_nonzero(kp) == hkv * d and np.count_nonzero(vp) == hkv * d


def test_store_writes_only_its_slots_and_skips_negative():
    rng = np.random.default_rng(0)
    nb, hkv, d, bs = 5, 2, 16, 4
    kp, vp = oracle.new_pools(nb, hkv, d, bs, POISON)
    n = 7
    slots = rng.choice(nb * bs, size=n, replace=False).astype(np.int32)
    slots[2] = -1
    slots[5] = -7
    k_new, v_new = rand_bits(rng, (n, hkv, d)), rand_bits(rng, (n, hkv, d))
    oracle.store_kv(kp, vp, k_new, v_new, slots)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, row = divmod(int(s), bs)
        written.add((blk, row))
        got_k = kp[blk, :, :, row, :].reshape(hkv, d)
        assert np.array_equal(got_k, k_new[i]) and np.array_equal(vp[blk, :, row, :], v_new[i])
    for blk in range(nb):
        for row in range(bs):
            if (blk, row) not in written:
                assert np.all(kp[blk, :, :, row, :] == POISON)
                assert np.all(vp[blk, :, row, :] == POISON)


def test_copy_blocks_moves_whole_blocks_and_skips_invalid_pairs():
    """Tokens stored into the source blocks read back, through a table that
    points at the destinations, exactly; untouched blocks keep their bytes;
    pairs with a negative or out-of-pool index or src == dst do nothing."""
    rng = np.random.default_rng(11)
    nb, hkv, d, bs = 6, 2, 16, 4
    kp, vp = oracle.new_pools(nb, hkv, d, bs, POISON)
    n = 2 * bs  # fill blocks 0 and 2 completely
    slots = np.concatenate([np.arange(0, bs), np.arange(2 * bs, 3 * bs)]).astype(np.int32)
    k_new, v_new = rand_bits(rng, (n, hkv, d)), rand_bits(rng, (n, hkv, d))
    oracle.store_kv(kp, vp, k_new, v_new, slots)
    k_before, v_before = kp.copy(), vp.copy()
    oracle.copy_blocks(kp, vp, [[0, 4], [2, 5], [-1, 1], [1, 1], [6, 3], [0, -2]])
    kg, vg = oracle.gather_seq(kp, vp, np.array([4, 5], np.int32), n)
    assert np.array_equal(kg, k_new) and np.array_equal(vg, v_new)
    for blk in (0, 1, 2, 3):
        assert np.array_equal(kp[blk], k_before[blk]) and np.array_equal(vp[blk], v_before[blk])
    assert np.all(kp[1] == POISON) and np.all(vp[3] == POISON)


def test_store_then_gather_round_trip():
    case = small_case(11, [1, 3, 4, 5, 9], 4, 2)
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    for b in range(case.batch):
        lo, hi = case.kv_offsets[b], case.kv_offsets[b + 1]
        kb, vb = oracle.gather_seq(kp, vp, case.block_table[b], int(case.context_lens[b]))
        assert np.array_equal(kb, k[lo:hi]) and np.array_equal(vb, v[lo:hi])


# ---------------------------------------------------------------- closed forms

def _golden_case(c):
    d = 8
    hq, hkv, bs = c["num_q_heads"], c["num_kv_heads"], c["block_size"]
    table = np.array(c["block_table"], np.int32)
    ctx = np.array(c["context_lens"], np.int32)
    kp, vp = oracle.new_pools(c["num_blocks"], hkv, d, bs, POISON)
    if "decoy_block" in c:
        dk = np.tile(f2bf(c["decoy_key"]), (1, hkv, 1))
        dv = np.tile(f2bf(c["decoy_value"]), (1, hkv, 1))
        oracle.store_kv(kp, vp, dk, dv, np.array([c["decoy_block"] * bs], np.int32))
    keys, vals = f2bf(c["keys"]), f2bf(c["values"])
    slots = [table[0, p // bs] * bs + p % bs for p in range(int(ctx[0]))]
    oracle.store_kv(kp, vp, keys, vals, np.array(slots, np.int32))
    return f2bf(c["q"]), kp, vp, table, ctx


def test_closed_form_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_cases.json")))
    for c in g["cases"]:
        q, kp, vp, table, ctx = _golden_case(c)
        if c["kind"] == "decode":
            got = oracle.decode(q, kp, vp, table, ctx, g["scale"])
        else:
            cu = np.array([0, c["q_lens"][0]], np.int32)
            got = oracle.prefill(q, cu, ctx, kp, vp, table, g["scale"])
        np.testing.assert_allclose(got, np.array(c["expected"]), rtol=0, atol=g["tolerance"],
                                   err_msg=c["name"])


def test_context_of_one_returns_v_exactly():
    case = small_case(12, [1, 1, 1], 8, 2, d=32)
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            expect = oracle.bf16_to_f64(v[case.kv_offsets[b], h // case.group])
            assert np.array_equal(out[b, h], expect)


def test_prefill_first_row_is_first_value():
    case = small_case(13, [5, 9], 4, 4, kind="prefill")
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    cu = case.q_offsets.astype(np.int32)
    out = oracle.prefill(q, cu, case.context_lens, kp, vp, case.block_table, case.scale)
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            assert np.array_equal(out[cu[b], h], oracle.bf16_to_f64(v[case.kv_offsets[b], h]))


def test_equal_keys_and_zero_query_give_mean_of_values():
    rng = np.random.default_rng(14)
    case = small_case(14, [7, 13], 2, 1, d=16)
    _, _, v = case_tensors(case)
    k = np.tile(rand_bits(rng, (1, 1, 16)), (case.total_kv_rows, 1, 1))
    kp, vp = build_pools(case, k, v)
    q = rand_bits(rng, (case.batch, 2, 16))
    q[:, 1, :] = 0  # head 1: zero query
    out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    for b in range(case.batch):
        lo, hi = case.kv_offsets[b], case.kv_offsets[b + 1]
        mean = oracle.bf16_to_f64(v[lo:hi, 0]).mean(axis=0)
        np.testing.assert_allclose(out[b, 0], mean, rtol=0, atol=1e-14)
        np.testing.assert_allclose(out[b, 1], mean, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (16, 8), (32, 8), (8, 1)])
def test_decode_matches_torch_sdpa_on_contiguous_cache(hq, hkv):
    lens = [1, 2, 5, 16, 17, 40]
    case = small_case(20 + hq, lens, hq, hkv, d=32, bs=8)
    # contiguous placement: identity block table
    table = np.full_like(case.block_table, -1)
    pos = 0
    for b, n in enumerate(lens):
        nb = wl.blocks_for(n, 8)
        table[b, :nb] = np.arange(pos, pos + nb)
        pos += nb
    case.block_table = table
    case.__dict__.pop("slot_mapping_all", None)
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    g = hq // hkv
    for b, n in enumerate(lens):
        lo = case.kv_offsets[b]
        kd = oracle.bf16_to_f64(k[lo:lo + n]).transpose(1, 0, 2).repeat(g, axis=0)
        vd = oracle.bf16_to_f64(v[lo:lo + n]).transpose(1, 0, 2).repeat(g, axis=0)
        qd = oracle.bf16_to_f64(q[b])[:, None, :]
        ref = sdpa(qd, kd, vd, case.scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(2, 1), (16, 8)])
def test_prefill_matches_torch_causal_sdpa(hq, hkv):
    lens = [1, 3, 8, 21]
    case = small_case(30 + hq, lens, hq, hkv, d=16, bs=4, kind="prefill")
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    cu = case.q_offsets.astype(np.int32)
    out = oracle.prefill(q, cu, case.context_lens, kp, vp, case.block_table, case.scale)
    g = hq // hkv
    for b, n in enumerate(lens):
        lo = case.kv_offsets[b]
        kd = oracle.bf16_to_f64(k[lo:lo + n]).transpose(1, 0, 2).repeat(g, axis=0)
        vd = oracle.bf16_to_f64(v[lo:lo + n]).transpose(1, 0, 2).repeat(g, axis=0)
        qd = oracle.bf16_to_f64(q[cu[b]:cu[b + 1]]).transpose(1, 0, 2)
        ref = sdpa(qd, kd, vd, case.scale, causal=True).transpose(1, 0, 2)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_physical_block_permutation_is_bit_identical():
    case = small_case(40, [3, 4, 9, 12, 1], 4, 2, bs=4, extra_blocks=6)
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    ref = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    rng = np.random.default_rng(41)
    for _ in range(3):
        perm = rng.permutation(case.num_blocks).astype(np.int32)
        table = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1)
        case2 = wl.PagedCase(**{**{f: getattr(case, f) for f in
                                   ("name", "kind", "seed", "num_q_heads", "num_kv_heads",
                                    "head_dim", "block_size", "context_lens", "q_lens",
                                    "num_blocks", "scale", "q_mult")},
                                "block_table": table})
        kp2, vp2 = build_pools(case2, k, v)
        out = oracle.decode(q, kp2, vp2, table, case.context_lens, case.scale)
        assert np.array_equal(out, ref)


def test_reads_exactly_the_blocks_of_each_sequence():
    """256k+1 rule: a sequence of n tokens owns ceil(n/256) blocks; every other
    block and every row past n is NaN poison, and -1 pads the table."""
    case = wl.tiny_decode()
    assert [int((r >= 0).sum()) for r in case.block_table] == [1, 1, 1, 2]
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    assert np.all(np.isfinite(out))


def test_prefill_row_equals_decode_at_that_length():
    case = small_case(50, [11], 4, 2, d=16, bs=4, kind="prefill")
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    cu = case.q_offsets.astype(np.int32)
    pre = oracle.prefill(q, cu, case.context_lens, kp, vp, case.block_table, case.scale)
    for i in range(11):
        dec = oracle.decode(q[i:i + 1], kp, vp, case.block_table, np.array([i + 1]), case.scale)
        # equal up to summation order (the prefill product also spans masked keys)
        np.testing.assert_allclose(dec[0], pre[i], rtol=0, atol=1e-14)


def test_split_merge_over_any_partition_equals_unsplit():
    rng = np.random.default_rng(60)
    for trial in range(20):
        n = int(rng.integers(1, 300))
        d = 16
        q = oracle.bf16_to_f64(rand_bits(rng, (3, d), scale=1 + 10 * (trial % 3)))
        k = oracle.bf16_to_f64(rand_bits(rng, (n, d)))
        v = oracle.bf16_to_f64(rand_bits(rng, (n, d)))
        ref = oracle.attend(q, k, v, 0.25)
        cuts = np.sort(rng.integers(0, n + 1, size=int(rng.integers(0, 6))))
        bounds = [0, *cuts.tolist(), n, n]  # repeated bounds give empty chunks
        parts = [oracle.split_partial(q, k[a:b], v[a:b], 0.25) for a, b in zip(bounds, bounds[1:])]
        np.testing.assert_allclose(oracle.merge_partials(parts), ref, rtol=0, atol=1e-12)


def test_empty_context_gives_zero_row():
    case = small_case(61, [0, 3], 2, 1)
    q, k, v = case_tensors(case)
    kp, vp = build_pools(case, k, v)
    out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1]))


# ---------------------------------------------------------------- brute force

def _brute(qv, ks, vs, scale):
    s = [scale * math.fsum(a * b for a, b in zip(qv, kk)) for kk in ks]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    return [math.fsum(e[j] * vs[j][dd] for j in range(len(ks))) / z for dd in range(len(qv))]


@pytest.mark.parametrize("bs", [1, 2, 3, 4])
def test_brute_force_tiny(bs):
    rng = np.random.default_rng(70 + bs)
    for trial in range(4):
        hkv = int(rng.integers(1, 3))
        hq = hkv * int(rng.choice([1, 2, 4]))
        d = 8 * int(rng.integers(1, 3))
        lens = [int(x) for x in rng.integers(1, 10, size=3)]
        kind = "prefill" if trial % 2 else "decode"
        # prefill rows: the last q_len of each context, q_len in 1..ctx (a
        # cached prefix of ctx - q_len tokens where q_len < ctx)
        q_lens = [int(rng.integers(1, n + 1)) for n in lens] if kind == "prefill" else None
        case = small_case(100 * bs + trial, lens, hq, hkv, d=d, bs=bs, kind=kind, q_lens=q_lens,
                          q_mult=float(2 ** int(rng.integers(0, 5))))
        q, k, v = case_tensors(case)
        kp, vp = build_pools(case, k, v)
        qf, kf, vf = (oracle.bf16_to_f64(x).tolist() for x in (q, k, v))
        if kind == "decode":
            out = oracle.decode(q, kp, vp, case.block_table, case.context_lens, case.scale)
        else:
            cu = case.q_offsets.astype(np.int32)
            out = oracle.prefill(q, cu, case.context_lens, kp, vp, case.block_table, case.scale)
        for b, n in enumerate(lens):
            lo = int(case.kv_offsets[b])
            qlen = int(case.q_lens[b])
            for i in range(qlen):
                pos = n - qlen + i
                row = b if kind == "decode" else int(case.q_offsets[b]) + i
                for h in range(hq):
                    g = h // (hq // hkv)
                    ks = [kf[lo + j][g] for j in range(pos + 1)]
                    vs = [vf[lo + j][g] for j in range(pos + 1)]
                    ref = _brute(qf[row][h], ks, vs, case.scale)
                    np.testing.assert_allclose(out[row, h], ref, rtol=0, atol=1e-13)
