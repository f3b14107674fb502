"""CPU oracle of the paged KV-cache path.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never does, and this package never imports them.
"""

from .block_manager import BlockManagerModel  # noqa: F401
from .paged_attention import (  # noqa: F401
    CHUNK,
    attend,
    bf16_to_f64,
    copy_blocks,
    decode,
    decode_seq,
    gather_seq,
    merge_partials,
    new_pools,
    prefill,
    prefill_seq,
    sparse_pools,
    split_partial,
    store_kv,
)
