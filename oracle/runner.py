"""Runs the oracle through one workload step. TEST INFRASTRUCTURE ONLY.

Given a workload from the seeded generators (any object with the same
attributes), builds the oracle's own caches by passing every request's
prior context through the oracle's slot mapping and cache write, then
applies the step's tokens the same way and computes the attention. Shares
no code with the HIP library.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import kvslot_oracle as O


class OracleStep:
    """Oracle state of one workload step.

    ``requests``: rows to materialise (default: every real request). With
    ``full_image`` the caches start as the generators' canary image, so the
    byte image after the writes can be compared whole; otherwise they start
    as (lazily allocated) zeros and only the chosen rows' blocks are written.
    """

    def __init__(self, w, table, requests=None, full_image=True, threads=1):
        self.w = w
        self.table = np.asarray(table, dtype=np.int32)
        self.rows = list(range(w.num_reqs)) if requests is None else \
            [int(r) for r in requests if 0 <= r < w.num_reqs]
        shape = (w.total_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        sd = {"f32": np.float32, "bf16": np.uint16}[w.dtype]
        if full_image:
            self.k_cache, self.v_cache = w.canary_cache(), w.canary_cache()
        else:
            self.k_cache, self.v_cache = np.zeros(shape, sd), np.zeros(shape, sd)
        self.step_parts = {}
        # the generators' draws of each request, ``threads`` at a time (each
        # request has its own random stream), then the oracle's own slot
        # mapping and cache write of its prior context, request by request
        with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
            draws = pool.map(w.request_kv, self.rows)
            for r, (k, v) in zip(self.rows, draws):
                c = int(w.computed[r])
                self.step_parts[r] = (k[c:], v[c:])
                if c:
                    req = np.full(c, r, np.int32)
                    pos = np.arange(c, dtype=np.int64)
                    slots = O.compute_slot_mapping(req, pos, self.table, w.block_size)
                    O.reshape_and_cache(k[:c], v[:c], slots, self.k_cache, self.v_cache)

    def step_tokens(self):
        """(req, pos, k, v) of the step: the ragged chunk, then the decode tokens."""
        w = self.w
        c_req, c_pos = w.chunk_tokens()
        d_req, d_pos = w.decode_tokens()
        req = np.concatenate([c_req, d_req])
        pos = np.concatenate([c_pos, d_pos])
        shape = (w.num_kv_heads, w.head_dim)
        sd = self.k_cache.dtype
        k = np.zeros((len(req), *shape), sd)
        v = np.zeros_like(k)
        for t, (r, p) in enumerate(zip(req, pos)):
            if r in self.step_parts:
                c = int(w.computed[r])
                k[t] = self.step_parts[r][0][p - c]
                v[t] = self.step_parts[r][1][p - c]
        return req, pos, k, v

    def write_step(self, max_num_tokens=None):
        """Slot mapping of every step token; writes only the materialised rows."""
        req, pos, k, v = self.step_tokens()
        slots = O.compute_slot_mapping(req, pos, self.table, self.w.block_size, max_num_tokens)
        mine = np.isin(req, self.rows)
        O.reshape_and_cache(k[mine], v[mine], slots[: len(req)][mine], self.k_cache, self.v_cache)
        return slots

    def attention(self, q, walk_blocks=None, requests=None, window=0, threads=1):
        """The oracle's attention of the chosen rows (default: the materialised
        ones); with ``threads`` > 1 the rows are spread over a thread pool, one
        request per call, and their outputs gathered."""
        w = self.w
        walk = self.table.shape[1] if walk_blocks is None else walk_blocks
        rows = self.rows if requests is None else list(requests)

        def run(rs):
            return O.paged_decode_attention(q, self.k_cache, self.v_cache, self.table,
                                            w.seq_lens, walk, w.scale, w.dtype, requests=rs,
                                            window=window)

        if threads <= 1 or len(rows) <= 1:
            return run(rows)
        out = None
        with ThreadPoolExecutor(max_workers=threads) as pool:
            for r, o in zip(rows, pool.map(lambda r: run([r]), rows)):
                if out is None:
                    out = np.zeros_like(o)
                out[r] = o[r]
        return out
