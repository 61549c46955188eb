"""ctypes binding of libkvslot.so: argument marshalling only.

Every function has the name of the C entry point it wraps (include/kvslot.h)
and runs no arithmetic of its own: tensors become device pointers, the
current torch stream becomes the hipStream_t, and a non-zero status becomes
KvslotError. PyTorch provides device memory and streams, nothing else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvslot.so")

KVS_OK = 0
KVS_F32, KVS_BF16 = 0, 1
KVS_WALK_TABLE = 0x1
STATUS = {
    0: "KVS_OK", -1: "KVS_EINVAL", -2: "KVS_EUNSUPPORTED", -3: "KVS_EBUCKET",
    -4: "KVS_ERANGE", -5: "KVS_ENOSPACE", -6: "KVS_EHIP",
}

# Every symbol include/kvslot.h declares.
EXPORTS = (
    "kvs_status_string",
    "kv_slot_mapping",
    "kv_cache_write",
    "kv_slot_mapping_cache_write",
    "select_ctx_bucket",
    "kv_map_to_kernel_blocks",
    "paged_decode_attention_workspace_bytes",
    "paged_decode_attention",
    "paged_decode_attention_noalloc",
    "paged_decode_attention_append",
    "paged_decode_attention_swa",
    "kv_swa_tail_trim",
    "kv_slot_mapping_dcp",
    "paged_decode_attention_dcp",
    "decode_lse_merge",
    "select_batch_bucket",
)


class KvslotError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name} ({_lib().kvs_status_string(status).decode()})")


_LIB = None


def _lib():
    """Load libkvslot.so once; fail loudly if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_slot_amd.build` "
                "(there is no fallback path)"
            )
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, u32, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        lib.kvs_status_string.argtypes = [ctypes.c_int]
        lib.kvs_status_string.restype = ctypes.c_char_p
        lib.kv_slot_mapping.argtypes = [vp, vp, i64, i64, vp, i32, i32, i32, vp, vp]
        lib.kv_cache_write.argtypes = [vp, vp, vp, i64, vp, vp, i64, i32, i32, i32, ctypes.c_int, vp]
        lib.kv_slot_mapping_cache_write.argtypes = [
            vp, vp, i64, i64, vp, i32, i32, i32, vp, vp, vp, vp, vp, i64, i32, i32, ctypes.c_int, vp,
        ]
        lib.select_ctx_bucket.argtypes = [i64, i32, vp, i32, i32, i32, vp, vp]
        lib.kv_map_to_kernel_blocks.argtypes = [vp, i32, i32, i32, i32, vp, i32]
        lib.paged_decode_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.paged_decode_attention_workspace_bytes.restype = sz
        lib.paged_decode_attention.argtypes = [
            vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32, i64, f32,
            ctypes.c_int, u32, vp, sz, vp, vp,
        ]
        lib.paged_decode_attention_noalloc.argtypes = [
            vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32, i64, f32,
            ctypes.c_int, u32, vp, vp,
        ]
        lib.paged_decode_attention_append.argtypes = [
            vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32,
            i32, i64, f32, ctypes.c_int, u32, vp, sz, vp, vp,
        ]
        lib.paged_decode_attention_swa.argtypes = [
            vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, f32,
            ctypes.c_int, vp, sz, vp, vp,
        ]
        lib.kv_swa_tail_trim.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp, i32, vp, vp]
        lib.kv_slot_mapping_dcp.argtypes = [vp, vp, i64, i64, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.paged_decode_attention_dcp.argtypes = [
            vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, i32, i32, i64, f32, ctypes.c_int,
            i32, i32, i32, vp, sz, vp, vp, vp,
        ]
        lib.decode_lse_merge.argtypes = [vp, vp, i32, i64, i32, vp, vp, vp]
        lib.select_batch_bucket.argtypes = [i32, vp, i32, vp]
        for name in ("kv_slot_mapping", "kv_cache_write", "kv_slot_mapping_cache_write",
                     "select_ctx_bucket", "kv_map_to_kernel_blocks", "paged_decode_attention",
                     "paged_decode_attention_noalloc", "paged_decode_attention_append",
                     "paged_decode_attention_swa", "kv_swa_tail_trim", "kv_slot_mapping_dcp",
                     "paged_decode_attention_dcp", "decode_lse_merge", "select_batch_bucket"):
            getattr(lib, name).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def load():
    """Load the library and return the ctypes handle."""
    return _lib()


def _check(status: int, where: str):
    if status != KVS_OK:
        raise KvslotError(status, where)


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out_shape(t: torch.Tensor, shape, where: str) -> None:
    """A caller-supplied output must have exactly the shape the call writes."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: out has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream)


def _kvs_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KVS_F32
    if t.dtype == torch.bfloat16:
        return KVS_BF16
    raise TypeError(f"unsupported cache dtype {t.dtype}")


def kv_slot_mapping(req_indices: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor,
                    block_size: int, slot_mapping: Optional[torch.Tensor] = None,
                    max_num_tokens: Optional[int] = None, stream=None) -> torch.Tensor:
    """Slots of the tokens (int64 [max_num_tokens]); see kv_slot_mapping in kvslot.h."""
    T = int(req_indices.numel())
    if slot_mapping is None:
        n = T if max_num_tokens is None else int(max_num_tokens)
        slot_mapping = torch.empty(n, dtype=torch.int64, device=block_table.device)
    rows, stride = block_table.shape
    st = _lib().kv_slot_mapping(
        _dev(req_indices, "req_indices", torch.int32, 1), _dev(positions, "positions", torch.int64, 1),
        T, int(slot_mapping.numel()), _dev(block_table, "block_table", torch.int32, 2),
        int(rows), int(stride), int(block_size), _dev(slot_mapping, "slot_mapping", torch.int64, 1),
        _stream(block_table, stream))
    _check(st, "kv_slot_mapping")
    return slot_mapping


def kv_cache_write(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
    """Scatter k_new / v_new [T, Hkv, D] into the caches in place; see kvslot.h."""
    nb, bs, hkv, d = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_new.shape[1:] != (hkv, d) \
            or v_new.shape != k_new.shape or k_new.dtype != k_cache.dtype \
            or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("kv_cache_write: shape or dtype mismatch")
    T = int(k_new.shape[0])
    if slot_mapping.numel() < T:
        raise ValueError("kv_cache_write: slot_mapping shorter than k_new")
    st = _lib().kv_cache_write(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int64),
        T, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), int(nb), int(bs), int(hkv), int(d),
        _kvs_dtype(k_cache), _stream(k_cache, stream))
    _check(st, "kv_cache_write")


def kv_slot_mapping_cache_write(req_indices: torch.Tensor, positions: torch.Tensor,
                                block_table: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                k_cache: torch.Tensor, v_cache: torch.Tensor,
                                slot_mapping: Optional[torch.Tensor] = None,
                                max_num_tokens: Optional[int] = None, stream=None) -> torch.Tensor:
    """kv_slot_mapping then kv_cache_write in one launch; returns the slots. See kvslot.h."""
    nb, bs, hkv, d = k_cache.shape
    T = int(req_indices.numel())
    if tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(k_new.shape) != (T, hkv, d) \
            or v_new.shape != k_new.shape or k_new.dtype != k_cache.dtype \
            or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise ValueError("kv_slot_mapping_cache_write: shape or dtype mismatch")
    if slot_mapping is None:
        n = T if max_num_tokens is None else int(max_num_tokens)
        slot_mapping = torch.empty(n, dtype=torch.int64, device=block_table.device)
    rows, stride = block_table.shape
    st = _lib().kv_slot_mapping_cache_write(
        _dev(req_indices, "req_indices", torch.int32, 1), _dev(positions, "positions", torch.int64, 1),
        T, int(slot_mapping.numel()), _dev(block_table, "block_table", torch.int32, 2),
        int(rows), int(stride), int(bs), _dev(slot_mapping, "slot_mapping", torch.int64, 1),
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        int(nb), int(hkv), int(d), _kvs_dtype(k_cache), _stream(k_cache, stream))
    _check(st, "kv_slot_mapping_cache_write")
    return slot_mapping


def select_ctx_bucket(max_num_computed_tokens: int, num_speculative_tokens: int,
                      buckets: Optional[Sequence[int]], max_model_len: int, block_size: int):
    """(bucket_len, walk_blocks) for this step; host only. See kvslot.h."""
    out_b, out_w = ctypes.c_int32(), ctypes.c_int32()
    if buckets is None:
        ptr, n, keep = None, 0, None
    else:
        keep = (ctypes.c_int32 * max(len(buckets), 1))(*[int(b) for b in buckets])
        ptr, n = ctypes.cast(keep, ctypes.c_void_p), len(buckets)
    st = _lib().select_ctx_bucket(int(max_num_computed_tokens), int(num_speculative_tokens), ptr, n,
                                  int(max_model_len), int(block_size), ctypes.byref(out_b),
                                  ctypes.byref(out_w))
    _check(st, "select_ctx_bucket")
    return out_b.value, out_w.value


def select_batch_bucket(num_active: int, buckets: Sequence[int]) -> int:
    """Padded batch size: the smallest bucket >= num_active; host only. See kvslot.h."""
    keep = (ctypes.c_int32 * max(len(buckets), 1))(*[int(b) for b in buckets])
    out = ctypes.c_int32()
    st = _lib().select_batch_bucket(int(num_active), ctypes.cast(keep, ctypes.c_void_p),
                                    len(buckets), ctypes.byref(out))
    _check(st, "select_batch_bucket")
    return out.value


def kv_map_to_kernel_blocks(block_table: np.ndarray, manager_block_size: int,
                            kernel_block_size: int) -> np.ndarray:
    """Expand a host block table from manager to kernel blocks; see kvslot.h."""
    src = np.ascontiguousarray(block_table, dtype=np.int32)
    rows, width = src.shape
    k = max(int(manager_block_size) // max(int(kernel_block_size), 1), 1)
    dst = np.empty((rows, width * k), dtype=np.int32)
    st = _lib().kv_map_to_kernel_blocks(src.ctypes.data, int(rows), int(width),
                                        int(manager_block_size), int(kernel_block_size),
                                        dst.ctypes.data, int(width * k))
    _check(st, "kv_map_to_kernel_blocks")
    return dst


def paged_decode_attention_workspace_bytes(num_seqs: int, q_len: int, num_q_heads: int,
                                           num_kv_heads: int, head_dim: int) -> int:
    return int(_lib().paged_decode_attention_workspace_bytes(
        int(num_seqs), int(q_len), int(num_q_heads), int(num_kv_heads), int(head_dim)))


def make_workspace(num_seqs: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                   head_dim: int, device) -> torch.Tensor:
    """A workspace of the required size (zero-filled, though the library needs
    no initial contents)."""
    n = paged_decode_attention_workspace_bytes(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim)
    if n == 0:
        raise ValueError("invalid sizes for the decode workspace")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                           walk_blocks: Optional[int] = None, flags: int = 0,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention; q [B, S_q, Hq, D] in the cache dtype -> fp32 out.

    walk_blocks defaults to the table width. See paged_decode_attention in
    kvslot.h for the semantics and the workspace contract.
    """
    B, Sq, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("paged_decode_attention: shape or dtype mismatch")
    if block_table.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("paged_decode_attention: block_table / seq_lens have too few rows")
    stride = int(block_table.shape[1])
    walk = stride if walk_blocks is None else int(walk_blocks)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    _out_shape(out, (B, Sq, Hq, D), "paged_decode_attention")
    if workspace is None:
        workspace = make_workspace(B, Sq, Hq, hkv, D, q.device)
    st = _lib().paged_decode_attention(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32, 2), stride, walk,
        _dev(seq_lens, "seq_lens", torch.int32), int(B), int(Sq), int(Hq), int(hkv), int(D),
        int(bs), int(nb), float(scale), _kvs_dtype(k_cache), int(flags),
        _dev(workspace, "workspace", torch.uint8), int(workspace.numel()),
        _dev(out, "out", torch.float32), _stream(q, stream))
    _check(st, "paged_decode_attention")
    return out


def paged_decode_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                                   walk_blocks: Optional[int] = None, flags: int = 0,
                                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """paged_decode_attention without a workspace: the library's own device
    array holds the split-K partials (calls on one GPU must not overlap).
    See paged_decode_attention_noalloc in kvslot.h."""
    B, Sq, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("paged_decode_attention_noalloc: shape or dtype mismatch")
    if block_table.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("paged_decode_attention_noalloc: block_table / seq_lens have too few rows")
    stride = int(block_table.shape[1])
    walk = stride if walk_blocks is None else int(walk_blocks)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    _out_shape(out, (B, Sq, Hq, D), "paged_decode_attention_noalloc")
    st = _lib().paged_decode_attention_noalloc(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32, 2), stride, walk,
        _dev(seq_lens, "seq_lens", torch.int32), int(B), int(Sq), int(Hq), int(hkv), int(D),
        int(bs), int(nb), float(scale), _kvs_dtype(k_cache), int(flags),
        _dev(out, "out", torch.float32), _stream(q, stream))
    _check(st, "paged_decode_attention_noalloc")
    return out


def paged_decode_attention_append(req_indices: torch.Tensor, positions: torch.Tensor,
                                  k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                                  k_cache: torch.Tensor, v_cache: torch.Tensor,
                                  block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                                  walk_blocks: Optional[int] = None, flags: int = 0,
                                  workspace: Optional[torch.Tensor] = None,
                                  out: Optional[torch.Tensor] = None,
                                  slot_mapping: Optional[torch.Tensor] = None,
                                  max_num_tokens: Optional[int] = None, stream=None):
    """The step's cache write and decode attention in one call; returns
    (slot_mapping, out). See paged_decode_attention_append in kvslot.h."""
    B, Sq, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("paged_decode_attention_append: shape or dtype mismatch")
    T = int(req_indices.numel())
    if positions.numel() != T or tuple(k_new.shape) != (T, hkv, D) \
            or tuple(v_new.shape) != (T, hkv, D) or k_new.dtype != k_cache.dtype \
            or v_new.dtype != k_cache.dtype:
        raise ValueError("paged_decode_attention_append: step token shapes or dtypes mismatch")
    if block_table.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("paged_decode_attention_append: block_table / seq_lens have too few rows")
    stride = int(block_table.shape[1])
    walk = stride if walk_blocks is None else int(walk_blocks)
    if slot_mapping is None:
        n = T if max_num_tokens is None else int(max_num_tokens)
        slot_mapping = torch.empty(n, dtype=torch.int64, device=q.device)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    _out_shape(out, (B, Sq, Hq, D), "paged_decode_attention_append")
    if workspace is None:
        workspace = make_workspace(B, Sq, Hq, hkv, D, q.device)
    st = _lib().paged_decode_attention_append(
        _dev(req_indices, "req_indices", torch.int32), _dev(positions, "positions", torch.int64),
        T, int(slot_mapping.numel()), _dev(slot_mapping, "slot_mapping", torch.int64),
        _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32, 2), stride, walk,
        _dev(seq_lens, "seq_lens", torch.int32), int(B), int(Sq), int(Hq), int(hkv), int(D),
        int(bs), int(nb), float(scale), _kvs_dtype(k_cache), int(flags),
        _dev(workspace, "workspace", torch.uint8), int(workspace.numel()),
        _dev(out, "out", torch.float32), _stream(q, stream))
    _check(st, "paged_decode_attention_append")
    return slot_mapping, out


def paged_decode_attention_swa(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                               sliding_window: int, kv_pos_offset: Optional[torch.Tensor] = None,
                               walk_blocks: Optional[int] = None,
                               workspace: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Sliding-window decode attention over a (tail-trimmed) table; see kvslot.h."""
    B, Sq, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("paged_decode_attention_swa: shape or dtype mismatch")
    if block_table.shape[0] < B or seq_lens.numel() < B or \
            (kv_pos_offset is not None and kv_pos_offset.numel() < B):
        raise ValueError("paged_decode_attention_swa: too few rows")
    stride = int(block_table.shape[1])
    walk = stride if walk_blocks is None else int(walk_blocks)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    _out_shape(out, (B, Sq, Hq, D), "paged_decode_attention_swa")
    if workspace is None:
        workspace = make_workspace(B, Sq, Hq, hkv, D, q.device)
    off = None if kv_pos_offset is None else _dev(kv_pos_offset, "kv_pos_offset", torch.int32, 1)
    st = _lib().paged_decode_attention_swa(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32, 2), stride, walk,
        _dev(seq_lens, "seq_lens", torch.int32), off, int(sliding_window), int(B), int(Sq), int(Hq),
        int(hkv), int(D), int(bs), int(nb), float(scale), _kvs_dtype(k_cache),
        _dev(workspace, "workspace", torch.uint8), int(workspace.numel()),
        _dev(out, "out", torch.float32), _stream(q, stream))
    _check(st, "paged_decode_attention_swa")
    return out


def kv_slot_mapping_dcp(req_indices: torch.Tensor, positions: torch.Tensor,
                        block_table: torch.Tensor, block_size: int, cp_world_size: int,
                        cp_rank: int, cp_interleave: int, slot_mapping: Optional[torch.Tensor] = None,
                        max_num_tokens: Optional[int] = None, stream=None) -> torch.Tensor:
    """Slots on one context-parallel rank (others' tokens -1); see kvslot.h."""
    T = int(req_indices.numel())
    if slot_mapping is None:
        n = T if max_num_tokens is None else int(max_num_tokens)
        slot_mapping = torch.empty(n, dtype=torch.int64, device=block_table.device)
    rows, stride = block_table.shape
    st = _lib().kv_slot_mapping_dcp(
        _dev(req_indices, "req_indices", torch.int32, 1), _dev(positions, "positions", torch.int64, 1),
        T, int(slot_mapping.numel()), _dev(block_table, "block_table", torch.int32, 2),
        int(rows), int(stride), int(block_size), int(cp_world_size), int(cp_rank), int(cp_interleave),
        _dev(slot_mapping, "slot_mapping", torch.int64, 1), _stream(block_table, stream))
    _check(st, "kv_slot_mapping_dcp")
    return slot_mapping


def paged_decode_attention_dcp(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                               cp_world_size: int, cp_rank: int, cp_interleave: int,
                               walk_blocks: Optional[int] = None,
                               workspace: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               stream=None):
    """One rank's attention over its keys; returns (out, lse). See kvslot.h."""
    B, Sq, Hq, D = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != D or q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("paged_decode_attention_dcp: shape or dtype mismatch")
    if block_table.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("paged_decode_attention_dcp: too few rows")
    stride = int(block_table.shape[1])
    walk = stride if walk_blocks is None else int(walk_blocks)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Sq, Hq), dtype=torch.float32, device=q.device)
    _out_shape(out, (B, Sq, Hq, D), "paged_decode_attention_dcp")
    _out_shape(lse, (B, Sq, Hq), "paged_decode_attention_dcp")
    if workspace is None:
        workspace = make_workspace(B, Sq, Hq, hkv, D, q.device)
    st = _lib().paged_decode_attention_dcp(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_table, "block_table", torch.int32, 2), stride, walk,
        _dev(seq_lens, "seq_lens", torch.int32), int(B), int(Sq), int(Hq), int(hkv), int(D), int(bs),
        int(nb), float(scale), _kvs_dtype(k_cache), int(cp_world_size), int(cp_rank),
        int(cp_interleave), _dev(workspace, "workspace", torch.uint8), int(workspace.numel()),
        _dev(out, "out", torch.float32), _dev(lse, "lse", torch.float32), _stream(q, stream))
    _check(st, "paged_decode_attention_dcp")
    return out, lse


def decode_lse_merge(outs: torch.Tensor, lses: torch.Tensor, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, stream=None):
    """Merge [world, ..., D] outputs and [world, ...] lse into (out, lse); see kvslot.h."""
    world = int(outs.shape[0])
    D = int(outs.shape[-1])
    rows = int(outs[0].numel()) // D if world else 0
    if tuple(lses.shape) != tuple(outs.shape[:-1]):
        raise ValueError("decode_lse_merge: lses must match outs without the last dim")
    if out is None:
        out = torch.empty(outs.shape[1:], dtype=torch.float32, device=outs.device)
    if lse is None:
        lse = torch.empty(lses.shape[1:], dtype=torch.float32, device=outs.device)
    _out_shape(out, outs.shape[1:], "decode_lse_merge")
    _out_shape(lse, lses.shape[1:], "decode_lse_merge")
    st = _lib().decode_lse_merge(_dev(outs, "outs", torch.float32), _dev(lses, "lses", torch.float32),
                                 world, rows, D, _dev(out, "out", torch.float32),
                                 _dev(lse, "lse", torch.float32), _stream(outs, stream))
    _check(st, "decode_lse_merge")
    return out, lse


def kv_swa_tail_trim(block_table: np.ndarray, seq_lens, q_len: int, sliding_window: int,
                     block_size: int):
    """Tail-trim a host block table for a sliding-window layer; see kvslot.h.

    Returns (trimmed table [rows, width] int32, kv_pos_offset [rows] int32).
    """
    src = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    rows, width = src.shape
    w = ctypes.c_int32()
    cap = max(width, 1)
    dst = np.empty((rows, cap), dtype=np.int32)
    off = np.empty(rows, dtype=np.int32)
    st = _lib().kv_swa_tail_trim(src.ctypes.data, int(rows), int(width), lens.ctypes.data,
                                 int(q_len), int(sliding_window), int(block_size), dst.ctypes.data,
                                 int(cap), off.ctypes.data, ctypes.byref(w))
    _check(st, "kv_swa_tail_trim")
    return np.ascontiguousarray(dst[:, : w.value]), off
