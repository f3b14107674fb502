"""Python binding of libpa.so, the gfx950 paged KV-cache attention library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors must be contiguous and live on the current HIP device; bf16
arrays may be passed as torch.bfloat16 or as int16 bit views.  Calls are
asynchronous on the current torch stream of the tensors' device (or on the
stream passed in).  The library must be built first
(``python -m paged_kv_cache_237_amd.build`` or ``__graft_entry__.build()``);
importing succeeds without it, and the first call raises if it is missing.

Cache layout (see include/pa.h): K cache bf16 [num_blocks, Hkv, 16, 256, 8],
V cache bf16 [num_blocks, Hkv, 256, 128].
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# PA_LIB_PATH selects another build of the library (the host-only sanitizer
# build that tests/test_host_sanitizers.py runs the CPU suites against).
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libpa.so")

BLOCK_SIZE = 256
HEAD_DIM = 128
K_CHUNK = 8

PA_OK = 0
STATUS_NAMES = {
    0: "PA_OK", -1: "PA_ERR_NULL_PTR", -2: "PA_ERR_BAD_SHAPE", -3: "PA_ERR_UNSUPPORTED",
    -4: "PA_ERR_ALIGN", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_HIP", -7: "PA_ERR_SLOT_RANGE",
    -8: "PA_ERR_DUPLICATE_SLOT", -9: "PA_ERR_BLOCK_CONFLICT", -10: "PA_ERR_NO_BLOCKS", -11: "PA_ERR_PRECONDITION",
}

EXPORTS = ("pa_store_kv", "pa_decode_workspace_size", "pa_decode", "pa_decode_append",
           "pa_decode_append_noalloc",
           "pa_decode_multi_workspace_size",
           "pa_decode_multi", "pa_prefill_workspace_size",
           "pa_prefill",
           "pa_copy_blocks", "pa_swap_blocks", "pa_validate_block_pairs",
           "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free", "pa_bm_allocate", "pa_bm_append",
           "pa_bm_append_batch", "pa_bm_fork", "pa_bm_free", "pa_bm_seq_len", "pa_bm_block_table", "pa_bm_slot_mapping",
           "pa_set_debug_checks", "pa_set_decode_waves", "pa_status_string", "pa_last_error_detail", "pa_validate_slots")


class PAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float


def lib() -> ctypes.CDLL:
    """The loaded library (torch's HIP runtime is loaded first so that libpa
    binds to that same runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m paged_kv_cache_237_amd.build` first")
        l = ctypes.CDLL(LIB_PATH)
        l.pa_store_kv.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _vp]
        l.pa_store_kv.restype = ctypes.c_int
        l.pa_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
        l.pa_decode_workspace_size.restype = _sz
        l.pa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i64, _f32, _vp, _sz, _vp]
        l.pa_decode.restype = ctypes.c_int
        l.pa_decode_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _i64, _f32, _vp, _sz, _vp]
        l.pa_decode_append.restype = ctypes.c_int
        l.pa_decode_append_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _i64, _f32, _vp]
        l.pa_decode_append_noalloc.restype = ctypes.c_int
        l.pa_decode_multi_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
        l.pa_decode_multi_workspace_size.restype = _sz
        l.pa_decode_multi.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _i64, _f32, _vp, _sz, _vp]
        l.pa_decode_multi.restype = ctypes.c_int
        l.pa_prefill_workspace_size.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
        l.pa_prefill_workspace_size.restype = _sz
        l.pa_prefill.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _vp, _i32, _i32,
                                 _i32, _i32, _i32, _i64, _f32, _vp, _sz, _vp]
        l.pa_prefill.restype = ctypes.c_int
        l.pa_set_decode_waves.argtypes = [_i32]
        l.pa_set_decode_waves.restype = ctypes.c_int
        l.pa_set_debug_checks.argtypes = [ctypes.c_int]
        l.pa_set_debug_checks.restype = ctypes.c_int
        l.pa_status_string.argtypes = [ctypes.c_int]
        l.pa_status_string.restype = ctypes.c_char_p
        l.pa_last_error_detail.argtypes = []
        l.pa_last_error_detail.restype = ctypes.c_char_p
        l.pa_validate_slots.argtypes = [_vp, _i64, _i64]
        l.pa_validate_slots.restype = ctypes.c_int
        l.pa_copy_blocks.argtypes = [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp]
        l.pa_copy_blocks.restype = ctypes.c_int
        l.pa_swap_blocks.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                     _vp]
        l.pa_swap_blocks.restype = ctypes.c_int
        l.pa_validate_block_pairs.argtypes = [_vp, _i64, _i64]
        l.pa_validate_block_pairs.restype = ctypes.c_int
        l.pa_bm_create.argtypes = [_i64, _i32]
        l.pa_bm_create.restype = _vp
        l.pa_bm_destroy.argtypes = [_vp]
        l.pa_bm_destroy.restype = None
        l.pa_bm_num_free.argtypes = [_vp]
        l.pa_bm_num_free.restype = _i64
        l.pa_bm_allocate.argtypes = [_vp, _i64, _i64]
        l.pa_bm_allocate.restype = ctypes.c_int
        l.pa_bm_append.argtypes = [_vp, _i64, _vp, _vp]
        l.pa_bm_append.restype = ctypes.c_int
        l.pa_bm_append_batch.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp]
        l.pa_bm_append_batch.restype = ctypes.c_int
        l.pa_bm_fork.argtypes = [_vp, _i64, _i64]
        l.pa_bm_fork.restype = ctypes.c_int
        l.pa_bm_free.argtypes = [_vp, _i64]
        l.pa_bm_free.restype = ctypes.c_int
        l.pa_bm_seq_len.argtypes = [_vp, _i64]
        l.pa_bm_seq_len.restype = _i64
        l.pa_bm_block_table.argtypes = [_vp, _vp, _i32, _vp, _i32]
        l.pa_bm_block_table.restype = ctypes.c_int
        l.pa_bm_slot_mapping.argtypes = [_vp, _i64, _i64, _i64, _vp]
        l.pa_bm_slot_mapping.restype = ctypes.c_int
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != PA_OK:
        raise PAError(status, lib().pa_last_error_detail().decode())


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16)
_I32 = (torch.int32,)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def alloc_cache(num_blocks: int, num_kv_heads: int, device="cuda", fill_bits: Optional[int] = None):
    """Allocate a (K, V) cache pair as bf16 tensors in the library layout,
    optionally filled with a bf16 bit pattern."""
    k = torch.empty((num_blocks, num_kv_heads, HEAD_DIM // K_CHUNK, BLOCK_SIZE, K_CHUNK),
                    dtype=torch.bfloat16, device=device)
    v = torch.empty((num_blocks, num_kv_heads, BLOCK_SIZE, HEAD_DIM), dtype=torch.bfloat16,
                    device=device)
    if fill_bits is not None:
        fb = fill_bits - 0x10000 if fill_bits >= 0x8000 else fill_bits
        k.view(torch.int16).fill_(fb)
        v.view(torch.int16).fill_(fb)
    return k, v


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    if k_cache.dim() != 5 or tuple(k_cache.shape[2:]) != (HEAD_DIM // K_CHUNK, BLOCK_SIZE, K_CHUNK):
        raise ValueError(f"k_cache must be [num_blocks, Hkv, 16, 256, 8], got {tuple(k_cache.shape)}")
    nb, hkv = int(k_cache.shape[0]), int(k_cache.shape[1])
    if tuple(v_cache.shape) != (nb, hkv, BLOCK_SIZE, HEAD_DIM):
        raise ValueError(f"v_cache must be [{nb}, {hkv}, 256, 128], got {tuple(v_cache.shape)}")
    return nb, hkv


def store_kv(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """pa_store_kv: k_new/v_new [N, Hkv, 128], slot_mapping int32 [N]."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    n = int(slot_mapping.shape[0])
    if tuple(k_new.shape) != (n, hkv, HEAD_DIM) or tuple(v_new.shape) != (n, hkv, HEAD_DIM):
        raise ValueError("k_new/v_new must be [N, Hkv, 128] matching slot_mapping and the cache")
    _check(lib().pa_store_kv(
        _dev(k_new, "k_new", _BF16), _dev(v_new, "v_new", _BF16),
        _dev(slot_mapping, "slot_mapping", _I32), n,
        _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16), nb, BLOCK_SIZE, hkv,
        HEAD_DIM, _stream(k_cache, stream)))


def decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int) -> int:
    n = lib().pa_decode_workspace_size(batch, num_q_heads, num_kv_heads, HEAD_DIM, BLOCK_SIZE)
    if n == 0 and batch > 0:
        raise PAError(-6, "pa_decode_workspace_size returned 0: " +
                      lib().pa_last_error_detail().decode())
    return int(n)


def alloc_decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, device="cuda"):
    """A zero-filled decode workspace (pa_decode resets its counters to zero,
    so it can be reused by later calls of the same or a smaller shape)."""
    n = decode_workspace_size(batch, num_q_heads, num_kv_heads)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def decode(out, q, k_cache, v_cache, block_table, context_lens, max_context_len: int,
           scale: float, workspace, stream=None) -> None:
    """pa_decode: q/out [B, Hq, 128], block_table int32 [B, max_blocks_per_seq],
    context_lens int32 [B]."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    b, hq, d = (int(x) for x in q.shape)
    if tuple(out.shape) != (b, hq, d) or block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("shape mismatch between q, out and block_table")
    if tuple(context_lens.shape) != (b,):
        raise ValueError("context_lens must be [B]")
    _check(lib().pa_decode(
        _dev(out, "out", _BF16), _dev(q, "q", _BF16), _dev(k_cache, "k_cache", _BF16),
        _dev(v_cache, "v_cache", _BF16), _dev(block_table, "block_table", _I32),
        int(block_table.shape[1]), _dev(context_lens, "context_lens", _I32), b,
        int(max_context_len), hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        _dev(workspace, "workspace", (torch.uint8, torch.float32, torch.int32)),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))


def decode_append(out, q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                  max_context_len: int, scale: float, workspace, stream=None) -> None:
    """pa_decode_append: pa_decode whose newest position of each sequence is
    the token k_new/v_new [B, Hkv, 128], which is also written into the
    caches at that position (one launch for the store and the decode)."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    b, hq, d = (int(x) for x in q.shape)
    if tuple(out.shape) != (b, hq, d) or block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("shape mismatch between q, out and block_table")
    if tuple(context_lens.shape) != (b,):
        raise ValueError("context_lens must be [B]")
    if tuple(k_new.shape) != (b, hkv, d) or tuple(v_new.shape) != (b, hkv, d):
        raise ValueError("k_new and v_new must be [B, Hkv, 128]")
    _check(lib().pa_decode_append(
        _dev(out, "out", _BF16), _dev(q, "q", _BF16), _dev(k_new, "k_new", _BF16),
        _dev(v_new, "v_new", _BF16), _dev(k_cache, "k_cache", _BF16),
        _dev(v_cache, "v_cache", _BF16), _dev(block_table, "block_table", _I32),
        int(block_table.shape[1]), _dev(context_lens, "context_lens", _I32), b,
        int(max_context_len), hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        _dev(workspace, "workspace", (torch.uint8, torch.float32, torch.int32)),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))


NOALLOC_SCRATCH_BYTES = 16777216


def decode_append_noalloc(out, q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                          max_context_len: int, scale: float, stream=None) -> None:
    """pa_decode_append_noalloc: pa_decode_append with the library's own
    per-device scratch instead of a workspace (nothing is allocated; calls
    that overlap in time on one device must not be made)."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    b, hq, d = (int(x) for x in q.shape)
    if tuple(out.shape) != (b, hq, d) or block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("shape mismatch between q, out and block_table")
    if tuple(context_lens.shape) != (b,):
        raise ValueError("context_lens must be [B]")
    if tuple(k_new.shape) != (b, hkv, d) or tuple(v_new.shape) != (b, hkv, d):
        raise ValueError("k_new and v_new must be [B, Hkv, 128]")
    _check(lib().pa_decode_append_noalloc(
        _dev(out, "out", _BF16), _dev(q, "q", _BF16), _dev(k_new, "k_new", _BF16),
        _dev(v_new, "v_new", _BF16), _dev(k_cache, "k_cache", _BF16),
        _dev(v_cache, "v_cache", _BF16), _dev(block_table, "block_table", _I32),
        int(block_table.shape[1]), _dev(context_lens, "context_lens", _I32), b,
        int(max_context_len), hq, hkv, d, BLOCK_SIZE, nb, float(scale), _stream(q, stream)))


def decode_multi_workspace_size(batch: int, q_per_seq: int, num_q_heads: int,
                                num_kv_heads: int) -> int:
    n = lib().pa_decode_multi_workspace_size(batch, q_per_seq, num_q_heads, num_kv_heads, HEAD_DIM,
                                             BLOCK_SIZE)
    if n == 0 and batch > 0:
        raise PAError(-3, "no workspace size for these shapes (q_per_seq * Hq/Hkv must be <= 32)")
    return int(n)


def alloc_decode_multi_workspace(batch: int, q_per_seq: int, num_q_heads: int, num_kv_heads: int,
                                 device="cuda"):
    """A zero-filled pa_decode_multi workspace (its counters are reset by
    every call, so it can be reused)."""
    n = decode_multi_workspace_size(batch, q_per_seq, num_q_heads, num_kv_heads)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def decode_multi(out, q, k_cache, v_cache, block_table, context_lens, q_per_seq: int,
                 max_context_len: int, scale: float, workspace, stream=None) -> None:
    """pa_decode_multi: q/out [B * q_per_seq, Hq, 128] (row b*q_per_seq + i),
    block_table int32 [B, max_blocks_per_seq], context_lens int32 [B]."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    rows, hq, d = (int(x) for x in q.shape)
    b = int(context_lens.shape[0])
    if tuple(out.shape) != (rows, hq, d) or rows != b * int(q_per_seq):
        raise ValueError("q and out must be [B * q_per_seq, Hq, head_dim]")
    if block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    _check(lib().pa_decode_multi(
        _dev(out, "out", _BF16), _dev(q, "q", _BF16), _dev(k_cache, "k_cache", _BF16),
        _dev(v_cache, "v_cache", _BF16), _dev(block_table, "block_table", _I32),
        int(block_table.shape[1]), _dev(context_lens, "context_lens", _I32), b, int(q_per_seq),
        int(max_context_len), hq, hkv, d, BLOCK_SIZE, nb, float(scale),
        _dev(workspace, "workspace", (torch.uint8, torch.float32, torch.int32)),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))


def prefill_workspace_size(batch: int, total_q_rows: int, max_seqlen_q: int, num_q_heads: int,
                           num_kv_heads: int, max_blocks_per_seq: int) -> int:
    return int(lib().pa_prefill_workspace_size(batch, total_q_rows, max_seqlen_q, num_q_heads,
                                               num_kv_heads, HEAD_DIM, BLOCK_SIZE, max_blocks_per_seq))


def alloc_prefill_workspace(batch: int, total_q_rows: int, max_seqlen_q: int, num_q_heads: int,
                            num_kv_heads: int, max_blocks_per_seq: int, device="cuda"):
    """A prefill workspace (scratch: no initial contents needed), or None
    when these sizes need none."""
    n = prefill_workspace_size(batch, total_q_rows, max_seqlen_q, num_q_heads, num_kv_heads,
                               max_blocks_per_seq)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def prefill(out, q, cu_seqlens_q, context_lens, max_seqlen_q: int, k_cache, v_cache,
            block_table, scale: float, workspace=None, stream=None) -> None:
    """pa_prefill: q/out [total_q, Hq, 128], cu_seqlens_q int32 [B+1] with
    cu_seqlens_q[B] = total_q, context_lens int32 [B], block_table int32
    [B, max_blocks_per_seq]; workspace from alloc_prefill_workspace."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    tq, hq, d = (int(x) for x in q.shape)
    b = int(context_lens.shape[0])
    if tuple(out.shape) != (tq, hq, d) or tuple(cu_seqlens_q.shape) != (b + 1,):
        raise ValueError("shape mismatch between q, out, cu_seqlens_q and context_lens")
    if block_table.dim() != 2 or block_table.shape[0] != b:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", (torch.uint8, torch.float32, torch.int32))
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().pa_prefill(
        _dev(out, "out", _BF16), _dev(q, "q", _BF16), _dev(cu_seqlens_q, "cu_seqlens_q", _I32),
        _dev(context_lens, "context_lens", _I32), b, int(max_seqlen_q), tq,
        _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(block_table, "block_table", _I32), int(block_table.shape[1]), hq, hkv, d,
        BLOCK_SIZE, nb, float(scale), ws_ptr, ws_bytes, _stream(q, stream)))


def set_debug_checks(enabled: bool) -> bool:
    """Turn the library's device-side precondition checks on or off (calls
    then synchronise their stream); returns the previous setting."""
    return bool(lib().pa_set_debug_checks(1 if enabled else 0))


def set_decode_waves(waves: int) -> int:
    """Testing aid: fix the number of runs the decode calls cut their work
    into (0 = automatic); returns the previous setting."""
    return int(lib().pa_set_decode_waves(int(waves)))


def validate_slots(slots_host, num_slots: int) -> int:
    """pa_validate_slots on a host int32 array; returns the status code."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(slots_host, dtype=np.int32))
    return int(lib().pa_validate_slots(arr.ctypes.data if arr.size else None, arr.size, num_slots))


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pa_copy_blocks: pairs int32 [n, 2] (src, dst) on the GPU."""
    nb, hkv = _cache_geometry(k_cache, v_cache)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    _check(lib().pa_copy_blocks(
        _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(pairs, "pairs", _I32), int(pairs.shape[0]), nb, BLOCK_SIZE, hkv, HEAD_DIM,
        _stream(k_cache, stream)))


def _pool_ptr(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _BF16:
        raise TypeError(f"{name} has dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs_host, stream=None) -> None:
    """pa_swap_blocks: copy whole blocks between two pools of the same layout
    (device or pinned host tensors); pairs_host is a host int32 [n, 2] array
    of (src block, dst block).  Asynchronous on the stream of the device
    pool."""
    import numpy as np
    snb, hkv = _cache_geometry(src_k, src_v)
    dnb, hkv2 = _cache_geometry(dst_k, dst_v)
    if hkv != hkv2:
        raise ValueError("pools have different kv head counts")
    arr = np.ascontiguousarray(np.asarray(pairs_host, dtype=np.int32).reshape(-1, 2))
    dev_t = src_k if src_k.is_cuda else dst_k
    _check(lib().pa_swap_blocks(
        _pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"), _pool_ptr(dst_k, "dst_k"),
        _pool_ptr(dst_v, "dst_v"), arr.ctypes.data if arr.size else None, arr.shape[0], snb, dnb,
        BLOCK_SIZE, hkv, HEAD_DIM, _stream(dev_t, stream)))


def validate_block_pairs(pairs_host, num_blocks: int) -> int:
    """pa_validate_block_pairs on a host int32 [n, 2] array; returns the status code."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(pairs_host, dtype=np.int32).reshape(-1, 2))
    return int(lib().pa_validate_block_pairs(arr.ctypes.data if arr.size else None, arr.shape[0],
                                             num_blocks))


class BlockManager:
    """The library's host block manager (pa_bm_*): fixed-size blocks with
    reference counts, on-demand growth at 256k+1 tokens, copy-on-write of a
    shared last block, fork and free; emits block tables and slot mappings."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        self._h = lib().pa_bm_create(num_blocks, block_size)
        if not self._h:
            raise PAError(-2, lib().pa_last_error_detail().decode())
        self._destroy = lib().pa_bm_destroy  # still callable at interpreter exit
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._destroy(h)
            self._h = None

    @property
    def num_free(self) -> int:
        return int(lib().pa_bm_num_free(self._h))

    def allocate(self, seq: int, num_tokens: int) -> None:
        _check(lib().pa_bm_allocate(self._h, seq, num_tokens))

    def append(self, seq: int):
        """One more token; returns (slot, copy_pair or None)."""
        slot = ctypes.c_int32(0)
        pair = (ctypes.c_int32 * 2)()
        _check(lib().pa_bm_append(self._h, seq, ctypes.byref(slot), pair))
        return int(slot.value), (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))

    def append_batch(self, seqs):
        """One token for each of seqs, all or nothing; returns (slots int32
        [n], copy pairs int32 [k, 2])."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = len(ids)
        slots = np.empty(n, dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        k = ctypes.c_int32(0)
        _check(lib().pa_bm_append_batch(self._h, ids.ctypes.data if n else None, n,
                                        slots.ctypes.data, pairs.ctypes.data, ctypes.byref(k)))
        return slots, pairs[:k.value].copy()

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pa_bm_fork(self._h, parent, child))

    def free(self, seq: int) -> None:
        _check(lib().pa_bm_free(self._h, seq))

    def seq_len(self, seq: int) -> int:
        return int(lib().pa_bm_seq_len(self._h, seq))

    def block_table(self, seqs, max_blocks_per_seq: int):
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        out = np.empty((len(ids), max_blocks_per_seq), dtype=np.int32)
        _check(lib().pa_bm_block_table(self._h, ids.ctypes.data if ids.size else None, len(ids),
                                       out.ctypes.data, max_blocks_per_seq))
        return out

    def slot_mapping(self, seq: int, first_pos: int, count: int):
        import numpy as np
        out = np.empty(count, dtype=np.int32)
        _check(lib().pa_bm_slot_mapping(self._h, seq, first_pos, count,
                                        out.ctypes.data if count else None))
        return out
