"""Plain Python model of the KV-cache block manager.  TEST INFRASTRUCTURE
ONLY (see the package docstring); it shares no code with the library.

Rules, from the pages:
  * nano-vllm hub page, "KV Cache block management": the cache is cut into
    blocks of a fixed 256 tokens, allocated and released with reference
    counts;
  * CSDN essay comparing nanoVLLM and vLLM, first section: each sequence has
    a block table of physical blocks, allocated on demand -- a new block is
    taken each time the sequence's length reaches 256k+1 (257, 513, ...).
Readings where the pages are silent (pinned in tests/test_block_manager.py):
  * a sequence that shares its last, not yet full block with another one
    takes a private copy before writing into it (copy-on-write), and reports
    the (shared, new) pair so that the block's contents can be copied;
  * free blocks are handed out first-in first-out from a queue that starts
    as 0, 1, ..., N-1; a block whose count drops to zero joins its end;
  * an operation that cannot be completed (unknown or existing sequence, too
    few free blocks) changes nothing.
"""

from __future__ import annotations

from collections import deque


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int = 256):
        self.block_size = block_size
        self.free = deque(range(num_blocks))
        self.ref = [0] * num_blocks
        self.seqs = {}  # seq id -> [length, [blocks]]

    def _take(self) -> int:
        b = self.free.popleft()
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def allocate(self, seq: int, num_tokens: int) -> bool:
        need = -(-num_tokens // self.block_size)
        if seq in self.seqs or num_tokens < 0 or need > len(self.free):
            return False
        self.seqs[seq] = [num_tokens, [self._take() for _ in range(need)]]
        return True

    def append(self, seq: int):
        """Returns (slot, copy pair or None), or None if it cannot."""
        if seq not in self.seqs:
            return None
        length, blocks = self.seqs[seq]
        pair = None
        if length % self.block_size == 0:
            if not self.free:
                return None
            blocks.append(self._take())
        elif self.ref[blocks[-1]] > 1:
            if not self.free:
                return None
            fresh = self._take()
            pair = (blocks[-1], fresh)
            self._release(blocks[-1])
            blocks[-1] = fresh
        self.seqs[seq][0] = length + 1
        return blocks[-1] * self.block_size + length % self.block_size, pair

    def append_batch(self, seqs):
        """append for each of seqs in turn; if one of them cannot, the state
        before the call is restored and None returned.  Otherwise (slots,
        copy pairs in the order they arose)."""
        if len(set(seqs)) != len(seqs) or any(s not in self.seqs for s in seqs):
            return None
        saved = (deque(self.free), list(self.ref),
                 {k: [v[0], list(v[1])] for k, v in self.seqs.items()})
        slots, pairs = [], []
        for s in seqs:
            r = self.append(s)
            if r is None:
                self.free, self.ref, self.seqs = saved
                return None
            slots.append(r[0])
            if r[1] is not None:
                pairs.append(r[1])
        return slots, pairs

    def fork(self, parent: int, child: int) -> bool:
        if parent not in self.seqs or child in self.seqs:
            return False
        length, blocks = self.seqs[parent]
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = [length, list(blocks)]
        return True

    def release(self, seq: int) -> bool:
        if seq not in self.seqs:
            return False
        for b in self.seqs.pop(seq)[1]:
            self._release(b)
        return True

    def table_row(self, seq: int, width: int):
        blocks = self.seqs[seq][1]
        return blocks + [-1] * (width - len(blocks))

    def slots(self, seq: int, first: int, count: int):
        blocks = self.seqs[seq][1]
        return [blocks[p // self.block_size] * self.block_size + p % self.block_size
                for p in range(first, first + count)]
