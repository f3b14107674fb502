"""Plain, slow CPU oracle of the paged KV-cache path (store, paged decode,
paged causal prefill).  TEST INFRASTRUCTURE ONLY: nothing on the product path
may import it; only the tests, the smoke check and the benchmark's CPU
baseline do.  It shares no code with the HIP library.

Arithmetic is float64 on the bf16 inputs (each bf16 value is widened exactly).
Caches and new K/V are handled as raw bf16 bit patterns (uint16), so the store
is a bit copy and can be compared byte for byte.

Cache layout (the library's ABI; the pages fix none):
  K pool: uint16 [num_blocks, Hkv, D/8, block_size, 8]
          element (slot, g, d) lives at [slot // bs, g, d // 8, slot % bs, d % 8]
  V pool: uint16 [num_blocks, Hkv, block_size, D]
          element (slot, g, d) lives at [slot // bs, g, slot % bs, d]

Sources (the pages; no code is taken from them):
  * nano-vllm hub page (pomoai.com), "Attention + Triton Kernel": new keys and
    values are written into preallocated cache blocks through a slot mapping.
  * same page, "KV Cache block management": blocks of a fixed 256 tokens.
  * CSDN essay comparing nanoVLLM and vLLM, first section (how the KV cache is
    managed): a block table maps each sequence's logical blocks to physical
    ones, which need not be contiguous; a sequence takes a new block on
    reaching 256k+1 tokens.
  * same essay, third section (how attention is computed): FlashAttention is
    exact attention reorganised to stay on chip, so the oracle is the plain
    definition softmax(scale * q K^T) V, per head.
  * same essay, reading vLLM's attention module: prefill and decode run as
    separate kernels; decode is one new token per sequence.

Readings where the pages are silent (each is a test-pinned choice):
  * grouped-query heads: q head h reads kv head h // (Hq / Hkv);
  * a negative slot means "do not store" (padding);
  * a new token is stored before it is attended, so decode attends to all
    context_lens[b] cached tokens, itself included;
  * prefill query row i of sequence b sits at absolute position
    ctx_b - q_len_b + i and sees keys 0..that position (bottom-right causal);
  * an empty context (ctx = 0) gives a zero output row.

Block copies (copy_blocks) follow the same bit-copy rule for whole blocks;
vLLM's swap between GPU and CPU memory moves whole blocks the same way.

Pins (tests/test_oracle.py): layout offsets written out by hand; store round
trip and untouched bytes; equality with torch's float64 scaled-dot-product
attention on contiguous caches; bit-identical results under any permutation
of physical blocks; ctx = 1 gives V exactly; equal keys give the mean of V;
hand-derived closed-form cases under tests/golden/; pure-Python brute force on
tiny shapes; prefill row i equals decode at ctx i+1; split-context merging
over any partition equals the unsplit result.
"""

from __future__ import annotations

import numpy as np

CHUNK = 8  # bf16 elements per 16-byte K chunk


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 pattern is the upper half of an IEEE float32."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int, fill: int):
    """Host pools in the library layout, every element holding ``fill``."""
    k = np.full((num_blocks, num_kv_heads, head_dim // CHUNK, block_size, CHUNK), fill, np.uint16)
    v = np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, np.uint16)
    return k, v


def sparse_pools(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int):
    """Zero pools whose pages are committed only when written (for large
    pools of which a test touches a few blocks)."""
    k = np.zeros((num_blocks, num_kv_heads, head_dim // CHUNK, block_size, CHUNK), np.uint16)
    v = np.zeros((num_blocks, num_kv_heads, block_size, head_dim), np.uint16)
    return k, v


def store_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             slot_mapping: np.ndarray) -> None:
    """Write token i's K/V (all kv heads) into cache slot slot_mapping[i].

    A bit copy: slot s is row s % bs of physical block s // bs.  Negative slots
    are skipped.  In place on the pools; tokens are taken in order.
    """
    nb, hkv, nchunk, bs, _ = k_pool.shape
    k_new = np.asarray(k_new, np.uint16)
    v_new = np.asarray(v_new, np.uint16)
    slots = np.asarray(slot_mapping, np.int64)
    for i in range(slots.shape[0]):
        s = int(slots[i])
        if s < 0:
            continue
        blk, row = divmod(s, bs)
        k_pool[blk, :, :, row, :] = k_new[i].reshape(hkv, nchunk, CHUNK)
        v_pool[blk, :, row, :] = v_new[i]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> None:
    """Copy whole blocks inside the pools: for each (src, dst) with both in
    range and src != dst, block dst (all kv heads, K and V) becomes a bit copy
    of block src.  Other pairs are skipped.  In place; the pairs are read in
    order, and a valid list writes no block twice and never reads a block it
    writes, so the order does not matter for it.  (CSDN essay, first section:
    blocks belong to sequences through the block table; a block shared by two
    sequences is copied before one of them writes to it.)"""
    nb = k_pool.shape[0]
    for src, dst in np.asarray(pairs, np.int64).reshape(-1, 2):
        if src < 0 or dst < 0 or src >= nb or dst >= nb or src == dst:
            continue
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def gather_seq(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray, n: int):
    """K and V bits [n, Hkv, D] of one sequence's positions 0..n-1, read
    through its block table: position p is row p % bs of physical block
    table_row[p // bs]."""
    nb, hkv, nchunk, bs, _ = k_pool.shape
    d = nchunk * CHUNK
    k = np.empty((n, hkv, d), np.uint16)
    v = np.empty((n, hkv, d), np.uint16)
    for lb in range((n + bs - 1) // bs):
        phys = int(table_row[lb])
        lo, hi = lb * bs, min(n, (lb + 1) * bs)
        rows = hi - lo
        kb = k_pool[phys, :, :, :rows, :]  # [Hkv, D/8, rows, 8]
        k[lo:hi] = kb.transpose(2, 0, 1, 3).reshape(rows, hkv, d)
        v[lo:hi] = v_pool[phys, :, :rows, :].transpose(1, 0, 2)
    return k, v


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
           last_pos: np.ndarray | None = None) -> np.ndarray:
    """softmax(scale * q k^T) v for query rows q [R, D] against keys k [n, D]
    and values v [n, D], all float64.  Row r sees keys 0..last_pos[r]
    (all keys when last_pos is None)."""
    r, n = q.shape[0], k.shape[0]
    if n == 0:
        return np.zeros((r, v.shape[1]), np.float64)
    s = (q @ k.T) * float(scale)
    if last_pos is not None:
        j = np.arange(n)[None, :]
        s = np.where(j <= np.asarray(last_pos)[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def decode_seq(q_bits: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
               table_row: np.ndarray, ctx: int, scale: float, heads=None) -> np.ndarray:
    """Decode output [Hq, D] (float64) for one sequence: every q head attends
    to all ctx cached tokens of its kv head.  ``heads`` limits the q heads
    computed (others are left as NaN)."""
    hq, d = q_bits.shape
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.full((hq, d), np.nan)
    heads = range(hq) if heads is None else heads
    if ctx <= 0:
        for h in heads:
            out[h] = 0.0
        return out
    kb, vb = gather_seq(k_pool, v_pool, table_row, ctx)
    q = bf16_to_f64(q_bits)
    for g in sorted({h // group for h in heads}):
        kg = bf16_to_f64(kb[:, g, :])
        vg = bf16_to_f64(vb[:, g, :])
        hs = [h for h in heads if h // group == g]
        out[hs] = attend(q[hs], kg, vg, scale)
    return out


def decode(q_bits: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
           context_lens: np.ndarray, scale: float) -> np.ndarray:
    """Paged decode, one query token per sequence: q bits [B, Hq, D] -> [B, Hq, D]."""
    return np.stack([decode_seq(q_bits[b], k_pool, v_pool, block_table[b], int(context_lens[b]),
                                scale) for b in range(q_bits.shape[0])]) \
        if q_bits.shape[0] else np.zeros(q_bits.shape, np.float64)


def prefill_seq(q_bits: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                table_row: np.ndarray, ctx: int, scale: float, heads=None,
                rows=None) -> np.ndarray:
    """Causal attention for one sequence's q_len query rows q_bits [q_len, Hq, D]
    over its ctx cached tokens; row i is at position ctx - q_len + i.
    ``heads``/``rows`` limit what is computed (the rest stays NaN)."""
    qlen, hq, d = q_bits.shape
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.full((qlen, hq, d), np.nan)
    heads = range(hq) if heads is None else heads
    rows = np.arange(qlen) if rows is None else np.asarray(rows)
    if qlen == 0 or rows.size == 0:
        return out
    kb, vb = gather_seq(k_pool, v_pool, table_row, ctx)
    last = ctx - qlen + rows
    for g in sorted({h // group for h in heads}):
        kg = bf16_to_f64(kb[:, g, :])
        vg = bf16_to_f64(vb[:, g, :])
        for h in heads:
            if h // group != g:
                continue
            q = bf16_to_f64(q_bits[rows, h, :])
            out[rows, h, :] = attend(q, kg, vg, scale, last)
    return out


def prefill(q_bits: np.ndarray, cu_seqlens_q: np.ndarray, context_lens: np.ndarray,
            k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
            scale: float) -> np.ndarray:
    """Varlen causal prefill over the paged cache: q bits [sum q_len, Hq, D]."""
    out = np.zeros(q_bits.shape, np.float64)
    for b in range(len(context_lens)):
        lo, hi = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        out[lo:hi] = prefill_seq(q_bits[lo:hi], k_pool, v_pool, block_table[b],
                                 int(context_lens[b]), scale)
    return out


# ---- split-context reduction (the decode merge, stated on its own) ----------

def split_partial(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Unnormalised state of one context chunk for query rows q [R, D]:
    m = max score, l = sum exp(s - m), u = sum exp(s - m) v.  An empty chunk
    gives m = -inf, l = 0, u = 0."""
    r, d = q.shape[0], v.shape[1]
    if k.shape[0] == 0:
        return np.full(r, -np.inf), np.zeros(r), np.zeros((r, d))
    s = (q @ k.T) * float(scale)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ v


def merge_partials(parts) -> np.ndarray:
    """Combine chunk states (m_i, l_i, u_i) into softmax(s) v:
    M = max m_i, L = sum exp(m_i - M) l_i, o = sum exp(m_i - M) u_i / L.
    Chunks with m = -inf carry no weight."""
    ms = np.stack([p[0] for p in parts])  # [S, R]
    big = ms.max(axis=0)
    w = np.where(np.isfinite(ms), np.exp(ms - big[None, :]), 0.0)
    big_l = sum(w[i] * parts[i][1] for i in range(len(parts)))
    u = sum(w[i][:, None] * parts[i][2] for i in range(len(parts)))
    return u / big_l[:, None]
