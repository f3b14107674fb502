"""Serving steps driven end to end by the library's host block manager on the
GPU: prompts stored at the manager's slot mappings, sequences forked so that
they share blocks, then decode steps in which every sequence appends a token
(one pa_bm_append_batch call or one pa_bm_append per sequence; the
copy-on-write pairs applied with pa_copy_blocks before the new tokens are
stored), a sequence is freed and a new one reuses its blocks.  After every
step the paged decode over the manager's block tables must equal, to the
attention bar, the float64 oracle's attention over each sequence's logical
token list -- which knows nothing of blocks, slots or copies.  A second run
of the same sequence makes every decode step one pa_decode_append launch
(the store left to the kernel, at the slot it derives from the table)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_237_amd as pa
import workloads as wl
from paged_harness import compare

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 8, 128
SEED = 71


def token_rows(stream, first, count):
    """bf16 bits [count, HKV, D] of global tokens first..first+count-1."""
    w = HKV * D
    return wl.normal_bf16(SEED, stream, first * w, count * w).view(count, HKV, D)


class Serving:
    def __init__(self, num_blocks):
        self.bm = pa.BlockManager(num_blocks)
        self.k, self.v = pa.alloc_cache(num_blocks, HKV, "cuda", fill_bits=wl.POISON_BF16)
        self.tokens = {}      # seq -> global token ids, in order
        self.next_token = 0
        self.copies = 0

    def _store(self, ids, slots):
        k = torch.cat([token_rows(wl.STREAM_K, i, 1) for i in ids]).cuda()
        v = torch.cat([token_rows(wl.STREAM_V, i, 1) for i in ids]).cuda()
        pa.store_kv(k, v, torch.as_tensor(np.asarray(slots, np.int32)).cuda(), self.k, self.v)

    def prompt(self, seq, n):
        self.bm.allocate(seq, n)
        ids = list(range(self.next_token, self.next_token + n))
        self.next_token += n
        self.tokens[seq] = ids
        if n:
            self._store(ids, self.bm.slot_mapping(seq, 0, n))

    def fork(self, parent, child):
        self.bm.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])

    def free(self, seq):
        self.bm.free(seq)
        del self.tokens[seq]

    def append_all(self, batched, fused=False):
        """One token per sequence.  fused: the store is left to
        pa_decode_append (decode_and_check), which writes each token at the
        slot its block table gives for the newest position; the manager's
        slot for that token must be the same one."""
        ids, slots, pairs = [], [], []
        seqs = sorted(self.tokens)
        if batched:
            slots, pairs = self.bm.append_batch(seqs)
            slots, pairs = slots.tolist(), [tuple(p) for p in pairs.tolist()]
        else:
            for seq in seqs:
                slot, pair = self.bm.append(seq)
                slots.append(slot)
                if pair is not None:
                    pairs.append(pair)
        for seq in seqs:
            ids.append(self.next_token)
            self.tokens[seq].append(self.next_token)
            self.next_token += 1
        if pairs:
            self.copies += len(pairs)
            pa.copy_blocks(self.k, self.v, torch.as_tensor(np.asarray(pairs, np.int32)).cuda())
        if fused:
            self.pending = (ids, slots)
        else:
            self._store(ids, slots)

    def decode_and_check(self, step, fused=False):
        seqs = sorted(self.tokens)
        lens = [len(self.tokens[s]) for s in seqs]
        width = max(max(-(-n // pa.BLOCK_SIZE) for n in lens), 1)
        tab = self.bm.block_table(seqs, width)
        table = torch.from_numpy(tab).cuda()
        ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
        w = HQ * D
        q = wl.normal_bf16(SEED, wl.STREAM_Q, step * len(seqs) * w, len(seqs) * w)
        q = q.view(len(seqs), HQ, D)
        out = torch.empty((len(seqs), HQ, D), dtype=torch.bfloat16, device="cuda")
        ws = pa.alloc_decode_workspace(len(seqs), HQ, HKV)
        scale = D ** -0.5
        if fused:
            ids, slots = self.pending
            for n, row, slot in zip(lens, tab, slots):
                p = n - 1
                assert slot == int(row[p // pa.BLOCK_SIZE]) * pa.BLOCK_SIZE + p % pa.BLOCK_SIZE
            k_new = torch.cat([token_rows(wl.STREAM_K, i, 1) for i in ids]).cuda()
            v_new = torch.cat([token_rows(wl.STREAM_V, i, 1) for i in ids]).cuda()
            pa.decode_append(out, q.cuda(), k_new, v_new, self.k, self.v, table, ctx, max(lens),
                             scale, ws)
        else:
            pa.decode(out, q.cuda(), self.k, self.v, table, ctx, max(lens), scale, ws)
        torch.cuda.synchronize()
        ref = np.zeros((len(seqs), HQ, D))
        qf = oracle.bf16_to_f64(wl.bits_to_numpy(q))
        for b, s in enumerate(seqs):
            ids = self.tokens[s]
            kf = oracle.bf16_to_f64(wl.bits_to_numpy(torch.cat([token_rows(wl.STREAM_K, i, 1) for i in ids])))
            vf = oracle.bf16_to_f64(wl.bits_to_numpy(torch.cat([token_rows(wl.STREAM_V, i, 1) for i in ids])))
            for h in range(HQ):
                g = h // (HQ // HKV)
                ref[b, h] = oracle.attend(qf[b, h][None, :], kf[:, g], vf[:, g], scale)[0]
        got = oracle.bf16_to_f64(wl.bits_to_numpy(out.view(torch.int16)))
        return compare(got, ref, f"managed decode step {step}")


def test_manager_driven_steps_match_attention_over_logical_tokens():
    print(f"[block manager] seed={SEED} hq={HQ} hkv={HKV}", flush=True)
    # 14 blocks: the prompts and the first step's appends take blocks 0..10,
    # so the late prompt of 1000 tokens takes the last three free blocks and
    # the block that freeing sequence 0 returned, stale contents and all
    sv = Serving(num_blocks=14)
    for seq, n in [(0, 300), (1, 256), (2, 700), (3, 1)]:
        sv.prompt(seq, n)
    sv.fork(0, 10)     # shares a partial last block: copy-on-write on append
    sv.fork(2, 11)     # the same, three blocks shared
    sv.fork(1, 12)     # shares only a full block: a new block on append
    for step in range(4):
        sv.append_all(batched=step % 2 == 0)
        sv.decode_and_check(step)
        if step == 1:
            sv.free(0)
            sv.prompt(20, 1000)
    assert sv.copies == 2
    assert sv.bm.num_free == 0
    seqs = sorted(sv.tokens)
    used = set(sv.bm.block_table(seqs, 4).ravel().tolist()) - {-1}
    assert used == set(range(14))


def test_manager_driven_steps_with_the_one_launch_step():
    """The same serving sequence with every decode step run as one
    pa_decode_append launch: the manager's slot of each new token is the
    slot the kernel derives from the block table, copy-on-write copies come
    first, and the outputs match attention over the logical tokens; the
    tokens the fused calls stored are read back by the next steps."""
    print(f"[block manager, pa_decode_append] seed={SEED}", flush=True)
    sv = Serving(num_blocks=14)
    for seq, n in [(0, 300), (1, 256), (2, 700), (3, 1)]:
        sv.prompt(seq, n)
    sv.fork(0, 10)
    sv.fork(2, 11)
    sv.fork(1, 12)
    for step in range(4):
        sv.append_all(batched=step % 2 == 0, fused=True)
        sv.decode_and_check(step, fused=True)
        if step == 1:
            sv.free(0)
            sv.prompt(20, 1000)
    assert sv.copies == 2
    assert sv.bm.num_free == 0
