"""Device-side set-up of a workload through the library's own entry points.

Allocates the canary-filled caches on the GPU, uploads the block table,
context lengths and q, and writes every request's prior context into the
cache with the library's kv_slot_mapping and kv_cache_write (a prefill, not
timed). The step's own tokens (the ragged chunk and the decode tokens) are
returned on the device for the caller to run through the path.

No arithmetic of the path happens here: slots and cache rows are produced
by the HIP library.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

import decode_attention_slot_amd as K

from . import CANARY_BITS, Workload


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def upload_storage(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host storage array (float32 or bf16 bits as uint16) -> device tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)


def canary_cache(w: Workload, device) -> torch.Tensor:
    """[total_blocks, bs, Hkv, D]: null block 0 zeros, every other element NaN canary."""
    shape = (w.total_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    if w.dtype == "f32":
        c = torch.full(shape, CANARY_BITS["f32"], dtype=torch.int32, device=device).view(torch.float32)
    else:
        c = torch.full(shape, CANARY_BITS["bf16"], dtype=torch.int16, device=device).view(torch.bfloat16)
    c[0].zero_()
    return c


def kernel_block_table(w: Workload) -> np.ndarray:
    """The table the kernels walk; manager tables are expanded by the library."""
    if w.block_table is not None:
        return w.block_table
    return K.kv_map_to_kernel_blocks(w.mgr_block_table, w.mgr_block_size, w.block_size)


@dataclasses.dataclass
class DeviceStep:
    """Device tensors of one step. *_req/_pos/_k/_v are the step's token lists."""

    w: Workload
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    q: torch.Tensor
    chunk_req: torch.Tensor
    chunk_pos: torch.Tensor
    chunk_k: torch.Tensor
    chunk_v: torch.Tensor
    dec_req: torch.Tensor
    dec_pos: torch.Tensor
    dec_k: torch.Tensor
    dec_v: torch.Tensor
    host_table: np.ndarray

    @property
    def step_req(self):
        return torch.cat([self.chunk_req, self.dec_req])

    @property
    def step_pos(self):
        return torch.cat([self.chunk_pos, self.dec_pos])


def dcp_block_table(w: Workload, world: int) -> np.ndarray:
    """The table one context-parallel rank walks: request r keeps the first
    ceil(L / (world * bs)) ids of its row, one per virtual block of world * bs
    positions (every rank shares it); other entries are -1."""
    table = kernel_block_table(w).copy()
    bs = w.block_size
    for r in range(table.shape[0]):
        L = int(w.seq_lens[r])
        n = -(-L // (world * bs)) if L > 0 else 0
        table[r, n:] = np.where(table[r, n:] == 0, 0, -1)
    return table


def build(w: Workload, device="cuda", threads: int = 8, batch_tokens: int = 1 << 19,
          prefill: bool = True, caches=None, dcp=None) -> DeviceStep:
    """Allocate, upload and prefill; returns the step's device tensors.

    ``caches`` reuses a (k_cache, v_cache) pair of the right shape (refilled
    with the canary) instead of allocating new ones. ``dcp = (world, rank,
    interleave)`` builds one context-parallel rank: its table
    (dcp_block_table) and a cache holding only the tokens it stores, written
    through kv_slot_mapping_dcp.
    """
    device = torch.device(device)
    table = kernel_block_table(w) if dcp is None else dcp_block_table(w, dcp[0])
    if caches is None:
        kc, vc = canary_cache(w, device), canary_cache(w, device)
    else:
        kc, vc = caches
        fresh = canary_cache(w, device)
        kc.copy_(fresh)
        vc.copy_(fresh)
        del fresh
    bt = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)
    sl = torch.from_numpy(np.ascontiguousarray(w.seq_lens, dtype=np.int32)).to(device)
    q = upload_storage(w.q(), w.dtype, device)

    rows = list(range(w.num_reqs))
    chunk_parts, dec_parts = {}, {}
    pending = []  # (req, pos, k, v) host pieces of prior context awaiting upload
    pending_tokens = 0

    def flush():
        nonlocal pending, pending_tokens
        if not pending:
            return
        req = np.concatenate([p[0] for p in pending])
        pos = np.concatenate([p[1] for p in pending])
        k = np.concatenate([p[2] for p in pending])
        v = np.concatenate([p[3] for p in pending])
        d_req = torch.from_numpy(req).to(device)
        d_pos = torch.from_numpy(pos).to(device)
        if dcp is None:
            slots = K.kv_slot_mapping(d_req, d_pos, bt, w.block_size)
        else:
            slots = K.kv_slot_mapping_dcp(d_req, d_pos, bt, w.block_size, *dcp)
        K.kv_cache_write(upload_storage(k, w.dtype, device), upload_storage(v, w.dtype, device),
                         slots, kc, vc)
        pending, pending_tokens = [], 0

    def draw(r):
        return r, w.request_kv(r)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        for r, (kr, vr) in ex.map(draw, rows):
            c, n = int(w.computed[r]), int(w.chunk_lens[r])
            chunk_parts[r] = (kr[c:c + n], vr[c:c + n])
            dec_parts[r] = (kr[c + n:], vr[c + n:])
            if prefill and c > 0:
                pending.append((np.full(c, r, np.int32), np.arange(c, dtype=np.int64), kr[:c], vr[:c]))
                pending_tokens += c
                if pending_tokens >= batch_tokens:
                    flush()
    if prefill:
        flush()

    sd = {"f32": np.float32, "bf16": np.uint16}[w.dtype]
    shape = (w.num_kv_heads, w.head_dim)

    def cat(parts, order):
        arr = [parts[r] for r in order]
        k = np.concatenate([a[0] for a in arr]) if arr else np.zeros((0, *shape), sd)
        v = np.concatenate([a[1] for a in arr]) if arr else np.zeros((0, *shape), sd)
        return k, v

    c_req, c_pos = w.chunk_tokens()
    ck, cv = cat(chunk_parts, rows)
    d_req, d_pos = w.decode_tokens()
    dk, dv = cat(dec_parts, rows)
    if w.num_decode_pad_tokens:  # dummy tokens carry zero rows
        pad = np.zeros((w.num_decode_pad_tokens, *shape), sd)
        dk, dv = np.concatenate([dk, pad]), np.concatenate([dv, pad])
    assert len(ck) == len(c_req) and len(dk) == len(d_req)

    def up_i(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)

    torch.cuda.synchronize(device)
    return DeviceStep(
        w=w, k_cache=kc, v_cache=vc, block_table=bt, seq_lens=sl, q=q,
        chunk_req=up_i(c_req), chunk_pos=up_i(c_pos),
        chunk_k=upload_storage(ck, w.dtype, device), chunk_v=upload_storage(cv, w.dtype, device),
        dec_req=up_i(d_req), dec_pos=up_i(d_pos),
        dec_k=upload_storage(dk, w.dtype, device), dec_v=upload_storage(dv, w.dtype, device),
        host_table=np.ascontiguousarray(table, dtype=np.int32),
    )


def run_step(s: DeviceStep, walk_blocks: Optional[int] = None, flags: int = 0, workspace=None,
             out=None, slots_out=None, fused: bool = False):
    """One step on the device: slot map + write of the step's tokens, then attention.

    fused: one kv_slot_mapping_cache_write launch instead of kv_slot_mapping
    followed by kv_cache_write. Returns (slot_mapping of the step tokens,
    attention output).
    """
    w = s.w
    req = torch.cat([s.chunk_req, s.dec_req])
    pos = torch.cat([s.chunk_pos, s.dec_pos])
    k = torch.cat([s.chunk_k, s.dec_k])
    v = torch.cat([s.chunk_v, s.dec_v])
    if fused:
        slots = K.kv_slot_mapping_cache_write(req, pos, s.block_table, k, v, s.k_cache, s.v_cache,
                                              slot_mapping=slots_out)
    else:
        slots = K.kv_slot_mapping(req, pos, s.block_table, w.block_size, slot_mapping=slots_out)
        K.kv_cache_write(k, v, slots, s.k_cache, s.v_cache)
    o = K.paged_decode_attention(s.q, s.k_cache, s.v_cache, s.block_table, s.seq_lens, w.scale,
                                 walk_blocks=walk_blocks, flags=flags, workspace=workspace, out=out)
    return slots, o
