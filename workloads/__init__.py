"""Seeded synthetic inputs for the Block KV decode path.

This module is shared by the tests, the benchmark and the smoke check. It
produces inputs only: request lengths, block tables, token index arrays and
the Q/K/V values. It contains none of the arithmetic the path computes (no
slot formula, no cache scatter, no attention); those live on both sides of
the parity check, in the oracle and in the HIP library, independently.

Inputs follow the workloads the pages describe:

* the block pool of "Padding and Batching with Block KV", section "Block
  Structure" (1024 blocks of 64 tokens, 8 KV heads, head_dim 128);
* block allocation for actual tokens only (same page, "Padding Does NOT
  Allocate Blocks"): a request of L tokens owns ceil(L / block_size) blocks;
* null block 0 reserved and never handed out (same page, "Block ID 0 vs.
  Sentinel -1"); unused table entries hold -1;
* context-length buckets [4096, 8192, 16384] with max_model_len 131072
  ("Decode Context-Length Bucketing", section "Examples");
* multi-token decode with 1 + 3 tokens per request ("Padding and Batching
  with Block KV", section "Multi-Token Decode");
* a manager block size of 32 split into kernel blocks of 16 and padded table
  rows filled with the null block (the vLLM block-table notes, "design
  motivation" list).

Every random draw comes from numpy's PCG64 ``default_rng`` seeded with a
tuple that names the config seed and the request, so any single request can
be regenerated alone (the parity tests at full size rely on that).
Q/K/V are N(0, 1) in float32; bf16 data is the float32 draw rounded to
nearest-even by torch and carried as raw uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "make_workload",
    "CONFIG_NAMES",
    "CANARY_BITS",
    "to_storage",
    "storage_dtype",
    "element_size",
]

# The five configurations, in order (index 0 is the tiny one).
CONFIG_NAMES = (
    "tiny_fp32",
    "block_config_bf16",
    "ctx_bucketing",
    "large_batch_block_split",
    "ragged_spec_decode",
)

# Quiet-NaN canaries that fill every cache byte no write should touch.
CANARY_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0}


def storage_dtype(dtype: str):
    """numpy dtype used to carry cache elements of ``dtype`` as raw data."""
    return {"f32": np.float32, "bf16": np.uint16}[dtype]


def element_size(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> storage representation (float32, or bf16 bits as uint16).

    bf16 rounding is round-to-nearest-even, done by torch's own conversion.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    import torch

    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


# Stream tags inside one config seed.
_TAG_LEN, _TAG_PERM, _TAG_Q, _TAG_K, _TAG_V, _TAG_MISC = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.

    Attributes (B = rows of the block table, including padded rows):
      name, index        config name and position in CONFIG_NAMES
      seed               config seed
      dtype              "f32" or "bf16" (cache, new K/V and q)
      block_size         kernel block size (tokens per block the kernels see)
      total_blocks       blocks in the pool (kernel blocks)
      num_kv_heads, num_q_heads, head_dim
      q_len              query tokens per request this step (1 + num_spec)
      num_reqs           real requests; rows num_reqs..B-1 are padding
      computed           int64 [B] tokens already in the cache before the step
                         (0 for padded rows)
      chunk_lens         int64 [B] extra prefill-chunk tokens written this
                         step before the decode tokens (ragged mix)
      seq_lens           int32 [B] context length after the step
                         (computed + chunk + q_len; 0 for padded rows)
      block_table        int32 [B, W] kernel block table; None when the
                         table is given at manager granularity (each side
                         expands it with its own code)
      mgr_block_table    int32 [B, Wm] manager table, or None
      mgr_block_size     manager block size, or None
      max_model_len      longest context the table can address
      buckets            decode context-length buckets, or None
      scale              softmax scale 1/sqrt(head_dim)
    """

    name: str
    index: int
    seed: int
    dtype: str
    block_size: int
    total_blocks: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    q_len: int
    num_reqs: int
    computed: np.ndarray
    chunk_lens: np.ndarray
    seq_lens: np.ndarray
    block_table: Optional[np.ndarray]
    mgr_block_table: Optional[np.ndarray] = None
    mgr_block_size: Optional[int] = None
    max_model_len: int = 0
    buckets: Optional[list] = None
    num_decode_pad_tokens: int = 0
    scale: float = 0.0

    # ---- sizes -----------------------------------------------------------
    @property
    def num_rows(self) -> int:
        return int(len(self.seq_lens))

    @property
    def table_width(self) -> int:
        """Kernel-table width (columns)."""
        if self.block_table is not None:
            return int(self.block_table.shape[1])
        k = self.mgr_block_size // self.block_size
        return int(self.mgr_block_table.shape[1]) * k

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def es(self) -> int:
        return element_size(self.dtype)

    @property
    def row_elems(self) -> int:
        """Elements of one (token, all KV heads) row."""
        return self.num_kv_heads * self.head_dim

    # ---- values ----------------------------------------------------------
    def request_kv(self, r: int, start: int = 0, stop: Optional[int] = None):
        """K and V of request ``r`` for positions [start, stop), storage dtype.

        Shape [stop - start, num_kv_heads, head_dim]. Values depend only on
        (seed, r, position), so any range can be drawn alone.
        """
        L = int(self.seq_lens[r])
        stop = L if stop is None else stop
        assert 0 <= start <= stop <= L
        out = []
        for tag in (_TAG_K, _TAG_V):
            full = self._request_draw(r, tag, L)
            out.append(to_storage(full[start:stop], self.dtype))
        return out[0], out[1]

    def _request_draw(self, r: int, tag: int, L: int) -> np.ndarray:
        g = _rng(self.seed, tag, r)
        return g.standard_normal((L, self.num_kv_heads, self.head_dim), dtype=np.float32)

    def q(self) -> np.ndarray:
        """q [B, q_len, num_q_heads, head_dim] in storage dtype (padded rows too)."""
        g = _rng(self.seed, _TAG_Q)
        x = g.standard_normal(
            (self.num_rows, self.q_len, self.num_q_heads, self.head_dim), dtype=np.float32
        )
        return to_storage(x, self.dtype)

    # ---- token lists -----------------------------------------------------
    def prior_tokens(self, rows=None):
        """(req_indices int32, positions int64) of the context already cached."""
        rows = range(self.num_reqs) if rows is None else rows
        req, pos = [], []
        for r in rows:
            n = int(self.computed[r])
            req.append(np.full(n, r, np.int32))
            pos.append(np.arange(n, dtype=np.int64))
        return _cat(req, np.int32), _cat(pos, np.int64)

    def chunk_tokens(self):
        """(req_indices, positions) of the ragged prefill chunk of this step."""
        req, pos = [], []
        for r in range(self.num_reqs):
            c, n = int(self.computed[r]), int(self.chunk_lens[r])
            req.append(np.full(n, r, np.int32))
            pos.append(np.arange(c, c + n, dtype=np.int64))
        return _cat(req, np.int32), _cat(pos, np.int64)

    def decode_tokens(self):
        """(req_indices, positions) of the decode tokens of this step.

        q_len consecutive positions per real request, then
        ``num_decode_pad_tokens`` dummy tokens (request -1, position 0) as a
        padded decode batch has.
        """
        req, pos = [], []
        for r in range(self.num_reqs):
            start = int(self.computed[r] + self.chunk_lens[r])
            req.append(np.full(self.q_len, r, np.int32))
            pos.append(np.arange(start, start + self.q_len, dtype=np.int64))
        if self.num_decode_pad_tokens:
            req.append(np.full(self.num_decode_pad_tokens, -1, np.int32))
            pos.append(np.zeros(self.num_decode_pad_tokens, np.int64))
        return _cat(req, np.int32), _cat(pos, np.int64)

    def token_kv(self, req: np.ndarray, pos: np.ndarray):
        """K/V rows [T, Hkv, D] (storage dtype) for a token list; pads are zero."""
        T = len(req)
        sd = storage_dtype(self.dtype)
        k = np.zeros((T, self.num_kv_heads, self.head_dim), sd)
        v = np.zeros_like(k)
        order = np.argsort(req, kind="stable")
        req_s = req[order]
        for r in np.unique(req_s):
            if r < 0:
                continue
            idx = order[req_s == r]
            p = pos[idx]
            lo, hi = int(p.min()), int(p.max()) + 1
            kr, vr = self.request_kv(int(r), lo, hi)
            k[idx] = kr[p - lo]
            v[idx] = vr[p - lo]
        return k, v

    def canary_cache(self) -> np.ndarray:
        """One cache tensor [total_blocks, bs, Hkv, D]: block 0 zeros, rest canary."""
        sd = storage_dtype(self.dtype)
        c = np.empty((self.total_blocks, self.block_size, self.num_kv_heads, self.head_dim), sd)
        c.view(np.uint16 if sd == np.uint16 else np.uint32)[...] = CANARY_BITS[self.dtype]
        c[0] = 0
        return c


def _cat(parts, dtype):
    return np.concatenate(parts).astype(dtype) if parts else np.zeros(0, dtype)


def _allocate(perm: np.ndarray, nblocks: np.ndarray, width: int, fill: int) -> np.ndarray:
    """Hand out consecutive chunks of ``perm`` to requests (the scheduler's part).

    Request r receives the next nblocks[r] ids in order; the rest of its row is
    ``fill``.
    """
    B = len(nblocks)
    table = np.full((B, width), fill, np.int32)
    off = 0
    for r in range(B):
        n = int(nblocks[r])
        assert n <= width, (n, width)
        table[r, :n] = perm[off : off + n]
        off += n
    assert off <= len(perm)
    return table


def _blocks_for(lengths: np.ndarray, block_size: int) -> np.ndarray:
    """Blocks the scheduler allocates for actual tokens: ceil(L / block_size)."""
    return np.array([-(-int(L) // block_size) for L in lengths], np.int64)


def pad_batch(w: Workload, rows: int) -> Workload:
    """The same step with the batch padded to ``rows`` rows by dummy requests.

    [BKV] "Decode Batch Padding": dummy requests allocate no blocks and write
    nothing; each contributes q_len tokens with request index -1 and position
    0 (so their slots are -1), and here a null-block table row and context
    length 0, so attention skips them. Real rows and their draws are
    unchanged (q is drawn row-major, so the real rows keep their values).
    """
    extra = rows - w.num_rows
    assert extra >= 0
    z64, z32 = np.zeros(extra, np.int64), np.zeros(extra, np.int32)
    kw = dict(
        computed=np.concatenate([w.computed, z64]),
        chunk_lens=np.concatenate([w.chunk_lens, z64]),
        seq_lens=np.concatenate([w.seq_lens, z32]).astype(np.int32),
        num_decode_pad_tokens=w.num_decode_pad_tokens + extra * w.q_len,
    )
    if w.block_table is not None:
        kw["block_table"] = np.vstack([w.block_table, np.zeros((extra, w.block_table.shape[1]),
                                                              np.int32)])
    else:
        kw["mgr_block_table"] = np.vstack([w.mgr_block_table,
                                           np.zeros((extra, w.mgr_block_table.shape[1]), np.int32)])
    return dataclasses.replace(w, **kw)


def tp_share(w: Workload, tp: int) -> Workload:
    """One tensor-parallel rank's share of a workload: num_kv_heads / tp KV
    heads and the matching num_q_heads / tp query heads, as a rank holds them
    ([KVC] KVCacheConfig at tensor parallelism 2: 8 KV heads become 4)."""
    if tp < 1 or w.num_kv_heads % tp or w.num_q_heads % tp:
        raise ValueError(f"tp {tp} does not divide {w.num_kv_heads} KV heads")
    return dataclasses.replace(w, num_kv_heads=w.num_kv_heads // tp,
                               num_q_heads=w.num_q_heads // tp)


def make_workload(index: int, seed: Optional[int] = None, **kw) -> Workload:
    """Build config ``index`` (0..4) with ``seed`` (default 1000 + index).

    Keyword overrides: ``num_reqs`` (configs 1, 3, 4), ``forced_max_ctx``
    (config 2: clip the lognormal draw and pin its maximum), ``ctx_hi``
    (configs 1 and 3: upper end of the uniform context draw), ``num_spec``
    (config 3: speculative tokens decoded per request, default 0).
    """
    seed = 1000 + index if seed is None else seed
    builder = (_tiny, _block_config, _bucketing, _large_batch, _ragged_spec)[index]
    w = builder(seed, **kw)
    w.index, w.name = index, CONFIG_NAMES[index]
    w.scale = 1.0 / math.sqrt(w.head_dim)
    return w


def _tiny(seed, **kw):
    # 2 requests that prefill 3 and 100 tokens, then decode one token each.
    bs, total = 64, 32
    computed = np.array([3, 100], np.int64)
    seq = computed + 1
    perm = _rng(seed, _TAG_PERM).permutation(np.arange(1, total, dtype=np.int32))
    table = _allocate(perm, _blocks_for(seq, bs), 4, -1)
    return Workload(
        name="", index=0, seed=seed, dtype="f32", block_size=bs, total_blocks=total,
        num_kv_heads=2, num_q_heads=8, head_dim=64, q_len=1, num_reqs=2,
        computed=computed, chunk_lens=np.zeros(2, np.int64), seq_lens=seq.astype(np.int32),
        block_table=table, max_model_len=4 * bs,
    )


def _block_config(seed, num_reqs=12, ctx_hi=5000, **kw):
    bs, total, W = 64, 1024, 80
    g = _rng(seed, _TAG_LEN)
    computed = g.integers(1, ctx_hi + 1, size=num_reqs).astype(np.int64)
    seq = computed + 1
    nb = _blocks_for(seq, bs)
    assert nb.sum() <= total - 1
    perm = _rng(seed, _TAG_PERM).permutation(np.arange(1, total, dtype=np.int32))
    table = _allocate(perm, nb, W, -1)
    return Workload(
        name="", index=1, seed=seed, dtype="bf16", block_size=bs, total_blocks=total,
        num_kv_heads=8, num_q_heads=32, head_dim=128, q_len=1, num_reqs=num_reqs,
        computed=computed, chunk_lens=np.zeros(num_reqs, np.int64),
        seq_lens=seq.astype(np.int32), block_table=table, max_model_len=W * bs,
    )


def _bucketing(seed, forced_max_ctx=None, num_reqs=8, **kw):
    bs, max_model_len = 64, 131072
    W = max_model_len // bs
    g = _rng(seed, _TAG_LEN)
    z = g.standard_normal(num_reqs)
    # lognormal with median 4096; sigma 1 is a reading (the config gives none)
    computed = np.clip(np.rint(4096.0 * np.exp(z)), 1, max_model_len - 1).astype(np.int64)
    if forced_max_ctx is not None:
        computed = np.minimum(computed, forced_max_ctx)
        computed[int(np.argmax(computed))] = forced_max_ctx
    seq = computed + 1
    nb = _blocks_for(seq, bs)
    total = int(nb.sum()) + 1
    perm = _rng(seed, _TAG_PERM).permutation(np.arange(1, total, dtype=np.int32))
    table = _allocate(perm, nb, W, -1)
    return Workload(
        name="", index=2, seed=seed, dtype="bf16", block_size=bs, total_blocks=total,
        num_kv_heads=8, num_q_heads=32, head_dim=128, q_len=1, num_reqs=num_reqs,
        computed=computed, chunk_lens=np.zeros(num_reqs, np.int64),
        seq_lens=seq.astype(np.int32), block_table=table, max_model_len=max_model_len,
        buckets=[4096, 8192, 16384],
    )


def _large_batch(seed, num_reqs=256, num_pad_rows=8, ctx_lo=512, ctx_hi=8192, num_spec=0, **kw):
    # num_spec > 0: the same batch decoding 1 + num_spec causal tokens per
    # request (speculative decoding), e.g. 32 query rows per KV head at 3
    mgr_bs, kern_bs = 32, 16
    q_len = 1 + num_spec
    g = _rng(seed, _TAG_LEN)
    computed = g.integers(ctx_lo, ctx_hi + 1, size=num_reqs).astype(np.int64)
    seq = computed + q_len
    Wm = max(257, -(-(ctx_hi + q_len) // mgr_bs))
    nb = _blocks_for(seq, mgr_bs)
    mgr_total = int(nb.sum()) + 1
    perm = _rng(seed, _TAG_PERM).permutation(np.arange(1, mgr_total, dtype=np.int32))
    mgr = _allocate(perm, nb, Wm, -1)
    # padded rows (batch padded to a fixed size) hold only the null block
    B = num_reqs + num_pad_rows
    mgr_full = np.zeros((B, Wm), np.int32)
    mgr_full[:num_reqs] = mgr
    computed_full = np.zeros(B, np.int64)
    computed_full[:num_reqs] = computed
    seq_full = np.zeros(B, np.int32)
    seq_full[:num_reqs] = seq
    return Workload(
        name="", index=3, seed=seed, dtype="bf16", block_size=kern_bs,
        total_blocks=mgr_total * (mgr_bs // kern_bs),
        num_kv_heads=8, num_q_heads=64, head_dim=128, q_len=q_len, num_reqs=num_reqs,
        computed=computed_full, chunk_lens=np.zeros(B, np.int64), seq_lens=seq_full,
        block_table=None,
        mgr_block_table=mgr_full, mgr_block_size=mgr_bs, max_model_len=Wm * mgr_bs,
        num_decode_pad_tokens=num_pad_rows * q_len,
    )


def _ragged_spec(seed, num_reqs=64, new_tokens=8192, num_spec=3, **kw):
    bs, W = 64, 512
    g = _rng(seed, _TAG_LEN)
    computed = g.integers(0, 16384, size=num_reqs).astype(np.int64)
    # uniform multinomial weights are a reading (the config names none)
    chunk = _rng(seed, _TAG_MISC).multinomial(new_tokens, [1.0 / num_reqs] * num_reqs).astype(np.int64)
    q_len = 1 + num_spec
    seq = computed + chunk + q_len
    nb = _blocks_for(seq, bs)
    total = int(nb.sum()) + 1
    perm = _rng(seed, _TAG_PERM).permutation(np.arange(1, total, dtype=np.int32))
    table = _allocate(perm, nb, W, -1)
    return Workload(
        name="", index=4, seed=seed, dtype="bf16", block_size=bs, total_blocks=total,
        num_kv_heads=8, num_q_heads=32, head_dim=128, q_len=q_len, num_reqs=num_reqs,
        computed=computed, chunk_lens=chunk, seq_lens=seq.astype(np.int32),
        block_table=table, max_model_len=W * bs,
    )
