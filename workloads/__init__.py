"""Seeded synthetic inputs for the paged KV-cache path.

This module is shared by the tests and the benchmark: both the HIP path and the
CPU oracle are fed from here.  It holds none of the attention arithmetic.  It
only

* draws sequence lengths and the physical block assignment of every sequence
  (the job of a block manager that hands out fixed-size blocks on demand, as
  the nano-vllm hub page describes in "KV Cache block management", and the
  CSDN essay describes in its first section on KV-cache management: a block
  table maps logical blocks to physical ones, and a new block is taken when a
  sequence grows to 256k+1 tokens);
* derives every cached token's slot number from its block table;
* produces bf16 tensor values with a counter-based generator, so that any
  slice of any tensor can be regenerated bit-identically on the CPU or on the
  GPU without materialising the whole tensor.

Value generator: element ``i`` of stream ``s`` under seed ``seed`` is
``TABLE[mix(i, key(seed, s)) >> 16]`` where ``mix`` is an integer avalanche
hash (xor-shift / odd-multiply rounds on 32-bit words, computed in int64 so
that no product overflows) and ``TABLE`` holds the 65,536 equiprobable
quantiles of N(0, 1), each rounded to bf16 (round to nearest even).  The
result is a bf16 sample of N(0, 1) quantised to 2^16 levels; the extreme
levels are about +-4.3.  Only integer operations and a table lookup are used,
so torch on the CPU and torch on the GPU give the same bits.
"""

from __future__ import annotations

import dataclasses
import functools
import math
import statistics
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK_SIZE = 256
HEAD_DIM = 128
POISON_BF16 = 0x7FC0  # a quiet NaN in bf16: unwritten cache bytes hold this

STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3

_M32 = 0xFFFFFFFF
_CHUNK = 1 << 24


@functools.lru_cache(maxsize=1)
def _normal_table_np() -> np.ndarray:
    """bf16 bit patterns of the 65,536 mid-point quantiles of N(0, 1)."""
    nd = statistics.NormalDist()
    n = 1 << 16
    x = np.array([nd.inv_cdf((i + 0.5) / n) for i in range(n)], dtype=np.float64)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    bf = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return bf.astype(np.uint16)


_table_cache: dict = {}


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    t = _table_cache.get(key)
    if t is None:
        t = torch.from_numpy(_normal_table_np().view(np.int16).copy()).to(device)
        _table_cache[key] = t
    return t


def _key(seed: int, stream: int) -> int:
    return ((seed * 0x9E3779B1) ^ (stream * 0x85EBCA77) ^ 0x5BD1E995) & _M32


def _mix(idx: torch.Tensor, key: int) -> torch.Tensor:
    """32-bit avalanche hash of int64 indices; every product stays below 2^63."""
    x = (idx & _M32) ^ (((idx >> 32) * 0x61C88647) & _M32) ^ key
    x = ((x ^ (x >> 16)) * 0x7FEB352D) & _M32
    x = ((x ^ (x >> 15)) * 0x2C1B3C6D) & _M32
    x = ((x ^ (x >> 16)) * 0x297A2D39) & _M32
    return x ^ (x >> 15)


def normal_bf16(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """``count`` bf16 values (as an int16 bit tensor) of stream ``stream``,
    elements ``start .. start+count-1``."""
    out = torch.empty(count, dtype=torch.int16, device=device)
    table = _normal_table(device)
    key = _key(seed, stream)
    for lo in range(0, count, _CHUNK):
        n = min(_CHUNK, count - lo)
        idx = torch.arange(start + lo, start + lo + n, dtype=torch.int64, device=device)
        out[lo:lo + n] = table[_mix(idx, key) >> 16]
    return out


def scale_bf16_bits(bits: torch.Tensor, factor: float) -> torch.Tensor:
    """Multiply bf16 values by a power of two (exact for the generator's range)."""
    assert factor > 0 and math.log2(factor).is_integer()
    return (bits.view(torch.bfloat16) * factor).view(torch.int16)


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks a sequence of n tokens holds: one more each time it reaches
    block_size*k + 1 tokens."""
    return (n_tokens + block_size - 1) // block_size


def pool_size_with_headroom(used_blocks: int) -> int:
    """ceil(1.1 * used) in integer arithmetic: 10 % free blocks on top."""
    return (11 * used_blocks + 9) // 10


@dataclasses.dataclass
class PagedCase:
    """One batch for the paged path: lengths, block tables and value streams.

    Token rows: the K/V of every cached token form a virtual dense tensor
    [sum(context_lens), Hkv, D] in batch order; sequence b owns rows
    kv_offsets[b] .. kv_offsets[b+1]-1, position p of sequence b is row
    kv_offsets[b] + p.  Query rows: [sum(q_lens), Hq, D]; the q_lens[b] query
    rows of sequence b sit at positions context_lens[b] - q_lens[b] .. ctx-1.
    """

    name: str
    kind: str  # "decode" or "prefill"
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray  # int32 [B]
    q_lens: np.ndarray  # int32 [B]
    num_blocks: int
    block_table: np.ndarray  # int32 [B, max_blocks_per_seq]; -1 = no block
    scale: float
    q_mult: float = 1.0

    # ---- shapes ---------------------------------------------------------
    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @functools.cached_property
    def kv_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.context_lens.astype(np.int64))])

    @functools.cached_property
    def q_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens.astype(np.int64))])

    @property
    def total_kv_rows(self) -> int:
        return int(self.kv_offsets[-1])

    @property
    def total_q_rows(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def used_blocks(self) -> int:
        return int(sum(blocks_for(int(n), self.block_size) for n in self.context_lens))

    # ---- slots ------------------------------------------------------------
    def slots_of_seq(self, b: int) -> np.ndarray:
        """Slot of every position 0..ctx-1 of sequence b."""
        n = int(self.context_lens[b])
        p = np.arange(n, dtype=np.int64)
        blk = self.block_table[b, p // self.block_size].astype(np.int64)
        return (blk * self.block_size + p % self.block_size).astype(np.int32)

    @functools.cached_property
    def slot_mapping_all(self) -> np.ndarray:
        """Slots of all cached tokens, in row order of the virtual dense K/V."""
        if self.batch == 0:
            return np.zeros(0, np.int32)
        return np.concatenate([self.slots_of_seq(b) for b in range(self.batch)]).astype(np.int32)

    def _new_tokens(self, b: int) -> int:
        return int(min(self.q_lens[b], self.context_lens[b]))

    def step_rows(self) -> np.ndarray:
        """Rows written by the step's store: the q_lens[b] newest tokens of
        each sequence (one per non-empty sequence for decode)."""
        rows = [np.arange(self.kv_offsets[b + 1] - self._new_tokens(b), self.kv_offsets[b + 1])
                for b in range(self.batch)]
        return np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)

    def history_rows(self) -> np.ndarray:
        """Rows already cached before the step (placed before timing)."""
        rows = [np.arange(self.kv_offsets[b], self.kv_offsets[b + 1] - self._new_tokens(b))
                for b in range(self.batch)]
        return np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)

    # ---- values -----------------------------------------------------------
    def _rows(self, stream: int, start: int, count: int, device) -> torch.Tensor:
        w = self.num_kv_heads * self.head_dim
        flat = normal_bf16(self.seed, stream, start * w, count * w, device)
        return flat.view(count, self.num_kv_heads, self.head_dim)

    def k_rows(self, start: int, count: int, device="cpu") -> torch.Tensor:
        """int16 bf16 bits [count, Hkv, D] of rows start..start+count-1."""
        return self._rows(STREAM_K, start, count, device)

    def v_rows(self, start: int, count: int, device="cpu") -> torch.Tensor:
        return self._rows(STREAM_V, start, count, device)

    def q_rows(self, start: int, count: int, device="cpu") -> torch.Tensor:
        """int16 bf16 bits [count, Hq, D] of query rows start..start+count-1."""
        w = self.num_q_heads * self.head_dim
        bits = normal_bf16(self.seed, STREAM_Q, start * w, count * w, device)
        if self.q_mult != 1.0:
            bits = scale_bf16_bits(bits, self.q_mult)
        return bits.view(count, self.num_q_heads, self.head_dim)

    def q_all(self, device="cpu") -> torch.Tensor:
        return self.q_rows(0, self.total_q_rows, device)


# ---------------------------------------------------------------------------
# builders


def assign_blocks(rng: np.random.Generator, context_lens: Sequence[int], num_blocks: int,
                  block_size: int = BLOCK_SIZE, max_blocks_per_seq: Optional[int] = None
                  ) -> np.ndarray:
    """Shuffle the pool (a seeded permutation) and hand each sequence, in
    batch order, the next ceil(ctx/block_size) physical blocks."""
    need = [blocks_for(int(n), block_size) for n in context_lens]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {sum(need)}")
    width = max(need) if need else 0
    if max_blocks_per_seq is not None:
        if max_blocks_per_seq < width:
            raise ValueError("max_blocks_per_seq too small")
        width = max_blocks_per_seq
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(need), max(width, 1)), -1, dtype=np.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return table


def make_case(name: str, kind: str, seed: int, context_lens: Sequence[int], num_q_heads: int,
              num_kv_heads: int, q_lens: Optional[Sequence[int]] = None,
              num_blocks: Optional[int] = None, head_dim: int = HEAD_DIM,
              block_size: int = BLOCK_SIZE, scale: Optional[float] = None, q_mult: float = 1.0,
              rng: Optional[np.random.Generator] = None,
              max_blocks_per_seq: Optional[int] = None) -> PagedCase:
    ctx = np.asarray(context_lens, dtype=np.int32)
    if kind == "decode":
        # one query row per sequence, also for an empty context
        ql = np.ones_like(ctx)
    elif q_lens is None:
        ql = ctx.copy()
    else:
        ql = np.asarray(q_lens, dtype=np.int32)
        if np.any(ql > ctx):
            raise ValueError("q_len may not exceed the context length")
    used = sum(blocks_for(int(n), block_size) for n in ctx)
    if num_blocks is None:
        num_blocks = max(pool_size_with_headroom(used), 1)
    if rng is None:
        rng = np.random.default_rng(seed)
    table = assign_blocks(rng, ctx, num_blocks, block_size, max_blocks_per_seq)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PagedCase(name=name, kind=kind, seed=seed, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                     context_lens=ctx, q_lens=ql, num_blocks=int(num_blocks), block_table=table,
                     scale=float(scale), q_mult=q_mult)


def tiny_decode() -> PagedCase:
    """4 sequences of 1, 255, 256 and 257 tokens; 16 q / 8 kv heads; 8-block pool."""
    return make_case("tiny_decode", "decode", 1, [1, 255, 256, 257], 16, 8, num_blocks=8)


def qwen3_0_6b_decode() -> PagedCase:
    """Batch 64, lengths uniform on 512..4096 (inclusive); 16 q / 8 kv heads."""
    rng = np.random.default_rng(2)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return make_case("qwen3_0.6b_decode", "decode", 2, ctx, 16, 8, rng=rng)


def qwen3_4b_decode() -> PagedCase:
    """Batch 256, lognormal lengths (median 2048, sigma 1 in natural log),
    rounded then clipped to 64..32768; 32 q / 8 kv heads."""
    rng = np.random.default_rng(3)
    raw = np.exp(rng.normal(math.log(2048.0), 1.0, size=256))
    ctx = np.clip(np.round(raw), 64, 32768).astype(np.int64)
    return make_case("qwen3_4b_decode", "decode", 3, ctx, 32, 8, rng=rng)


def prefill_8x2048() -> PagedCase:
    """8 sequences x 2048 prompt tokens (16,384 tokens), 16 q / 8 kv heads;
    every token is stored then attended causally."""
    return make_case("prefill_8x2048", "prefill", 4, [2048] * 8, 16, 8)


def long_context_decode() -> PagedCase:
    """Batch 8, 131,072 tokens each (512 blocks per sequence); 32 q / 8 kv heads."""
    return make_case("long_context_decode", "decode", 5, [131072] * 8, 32, 8)


def chunked_prefill_mixed() -> PagedCase:
    """One step of chunked prefill mixed with decoding: 64 sequences decode one
    token over U{512..4096} cached tokens, and 8 sequences continue their prompt
    with a 512-token chunk on top of a cached prefix of U{512..8192} tokens
    (4,160 query rows); 16 q / 8 kv heads.  Decode rows come first in the
    batch."""
    rng = np.random.default_rng(6)
    dctx = rng.integers(512, 4096, size=64, endpoint=True)
    prefix = rng.integers(512, 8192, size=8, endpoint=True)
    ctx = np.concatenate([dctx, prefix + 512])
    ql = np.concatenate([np.ones(64, dtype=np.int64), np.full(8, 512, dtype=np.int64)])
    return make_case("chunked_prefill_mixed", "prefill", 6, ctx, 16, 8, q_lens=ql, rng=rng)


def multi_query_decode() -> PagedCase:
    """Speculative verification: 64 sequences each score 4 new tokens (3
    drafted + 1) over U{512..4096} cached tokens, causally among themselves;
    16 q / 8 kv heads."""
    rng = np.random.default_rng(7)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return make_case("multi_query_decode", "prefill", 7, ctx, 16, 8,
                     q_lens=np.full(64, 4, dtype=np.int64), rng=rng)


def spec_verify_decode() -> PagedCase:
    """Speculative verification with 5 drafted tokens: 64 sequences each score
    the 5 drafted tokens and the next one (6 new tokens) over U{512..4096}
    cached tokens, causally among themselves; 16 q / 8 kv heads."""
    rng = np.random.default_rng(9)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return make_case("spec_verify_decode", "prefill", 9, ctx, 16, 8,
                     q_lens=np.full(64, 6, dtype=np.int64), rng=rng)


def spec_verify_decode_g4() -> PagedCase:
    """Speculative verification with 5 drafted tokens at 4 query heads per kv
    head: the batch of spec_verify_decode (64 sequences, 6 new tokens each
    over U{512..4096} cached tokens) with 32 q / 8 kv heads, so a (sequence,
    kv head) holds 24 query rows."""
    rng = np.random.default_rng(9)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return make_case("spec_verify_decode_g4", "prefill", 9, ctx, 32, 8,
                     q_lens=np.full(64, 6, dtype=np.int64), rng=rng)


def long_prefix_chunk() -> PagedCase:
    """One long prompt mid-way through chunked prefill: a 512-token chunk on
    top of a 65,536-token cached prefix, one sequence; 16 q / 8 kv heads."""
    return make_case("long_prefix_chunk", "prefill", 8, [65536 + 512], 16, 8, q_lens=[512])


def long_chunk_with_decode() -> PagedCase:
    """Chunked prefill beside a decode batch when one prompt is far longer
    than the rest: a 512-token chunk on top of a 32,768-token cached prefix
    and 63 sequences decoding one token over U{512..4096} cached tokens;
    16 q / 8 kv heads.  The chunk comes first in the batch."""
    rng = np.random.default_rng(33)
    dctx = rng.integers(512, 4096, size=63, endpoint=True)
    ctx = np.concatenate([[32768 + 512], dctx])
    ql = np.concatenate([[512], np.ones(63, dtype=np.int64)])
    return make_case("long_chunk_with_decode", "prefill", 33, ctx, 16, 8, q_lens=ql, rng=rng)


CONFIGS = {
    "tiny_decode": tiny_decode,
    "qwen3_0.6b_decode": qwen3_0_6b_decode,
    "qwen3_4b_decode": qwen3_4b_decode,
    "prefill_8x2048": prefill_8x2048,
    "long_context_decode": long_context_decode,
    "chunked_prefill_mixed": chunked_prefill_mixed,
    "multi_query_decode": multi_query_decode,
    "long_prefix_chunk": long_prefix_chunk,
    "spec_verify_decode": spec_verify_decode,
    "spec_verify_decode_g4": spec_verify_decode_g4,
    "long_chunk_with_decode": long_chunk_with_decode,
}


def bits_to_numpy(t: torch.Tensor) -> np.ndarray:
    """A bf16/int16 tensor (any device) as a host uint16 array of bf16 bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
