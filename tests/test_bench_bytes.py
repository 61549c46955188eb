"""The benchmark's algorithmic byte counts against an independent count.

Every roofline figure divides bytes by time, so the byte formulas in bench.py
are checked here by enumeration: the positions a walk must read are listed
one by one, the distinct (request, block) pairs they fall in are counted, and
the bytes are summed from the arrays' own sizes. CPU only.
"""

import glob
import json
import math
import os

import numpy as np
import pytest

import bench
import oracle as O
import workloads as W


def block_bytes(w):
    # one K block and one V block of every KV head, plus its table entry
    return 2 * w.block_size * w.num_kv_heads * w.head_dim * w.es + 4


def q_out_bytes(w):
    q = w.q()
    return q.size * w.es + q.size * 4  # q in the cache dtype, fp32 out of the same shape


def distinct_blocks(w, positions_of):
    return sum(len({p // w.block_size for p in positions_of(r)}) for r in range(w.num_rows))


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_context_walk_bytes(index):
    w = W.make_workload(index)
    width = w.table_width
    lens = [int(x) for x in w.seq_lens]
    n = distinct_blocks(w, lambda r: range(max(lens[r], 0)))
    want = n * block_bytes(w) + q_out_bytes(w) + 4 * w.num_rows
    assert bench.attention_bytes(w, width, table_walk=False) == want
    # token-exact lower bound: the rows of the visible positions only
    row = 2 * w.num_kv_heads * w.head_dim * w.es
    exact = sum(lens) * row + 4 * n + q_out_bytes(w) + 4 * w.num_rows
    assert bench.attention_bytes_token_exact(w, width) == exact


@pytest.mark.parametrize("walk", [64, 256, 2048])
def test_table_walk_and_head_trim_bytes(walk):
    w = W.make_workload(2)
    lens = [int(x) for x in w.seq_lens]
    # fixed-shape walk: every walked column of every row
    want_table = w.num_rows * walk * block_bytes(w) + q_out_bytes(w) + 4 * w.num_rows
    assert bench.attention_bytes(w, walk, table_walk=True) == want_table
    # context walk with a head trim: positions below the trimmed width only
    n = distinct_blocks(w, lambda r: range(min(lens[r], walk * w.block_size)))
    want = n * block_bytes(w) + q_out_bytes(w) + 4 * w.num_rows
    assert bench.attention_bytes(w, walk, table_walk=False) == want


@pytest.mark.parametrize("window", [1, 100, 4096])
def test_window_bytes(window):
    w = W.make_workload(4)
    table = w.block_table
    lens = w.seq_lens[: w.num_rows].astype(np.int32)
    trimmed, off = O.swa_tail_trim(table, lens, w.q_len, window, w.block_size)
    width = trimmed.shape[1]

    def visible(r):
        # keys some query of the step sees, inside the trimmed frame
        L = int(lens[r])
        lo = max(int(off[r]), L - w.q_len - window + 1)
        hi = min(L, int(off[r]) + width * w.block_size)
        return range(lo, hi)

    n = distinct_blocks(w, visible)
    # q, out, seq_len and the per-request offset
    want = n * block_bytes(w) + q_out_bytes(w) + 8 * w.num_rows
    assert bench.window_attention_bytes(w, window, off, width) == want


@pytest.mark.parametrize("world,rank,interleave", [(2, 0, 1), (4, 1, 1), (4, 3, 16)])
def test_context_parallel_share_bytes(world, rank, interleave):
    w = W.make_workload(4)
    lens = [int(x) for x in w.seq_lens]

    def local_positions(r):
        ps = np.arange(lens[r])
        mine = ps[O.dcp_owner(ps, world, interleave) == rank]
        return [int(x) for x in O.dcp_local_position(mine, world, interleave)]

    n = distinct_blocks(w, local_positions)
    rows = w.num_rows * w.q_len * w.num_q_heads
    # q in, fp32 out and lse, seq_len
    want = (n * block_bytes(w) + rows * w.head_dim * (w.es + 4) + 4 * rows + 4 * w.num_rows)
    assert bench.dcp_attention_bytes(w, world, rank, interleave) == want


def test_step_write_bytes():
    w = W.make_workload(3)
    T = w.num_reqs * w.q_len + w.num_decode_pad_tokens
    live = w.num_reqs * w.q_len
    # each written token reads and writes its K and V rows; every slot is read
    row = w.num_kv_heads * w.head_dim * w.es
    assert bench.cache_write_bytes(w, live, T) == live * 4 * row + 8 * T
    assert bench.slot_map_bytes(T) == 24 * T
    assert math.isclose(bench.slot_map_bytes(1 << 22) / (1 << 22), 24.0)


def test_committed_counter_traffic_is_for_these_kernels():
    """Every committed pass-1 counter summary was taken with the decode kernels
    as they are (the hash of their code), so the bench line's traffic for the
    256-request step resolves instead of being dropped as stale; and there the
    DRAM bytes are within a few percent of the algorithmic bytes of the call."""
    paths = sorted(glob.glob(os.path.join(bench.ROOT, "profiles",
                                          "paged_decode_attention_*_traffic.json")))
    assert paths
    for path in paths:
        with open(path) as f:
            d = json.load(f)
        assert d["kernel_source_sha256_16"] == bench.kernel_source_hash(), path
    t = bench.measured_traffic("large_batch_block_split", "context")
    assert t is not None
    with open(os.path.join(bench.ROOT, "profiles",
                           "paged_decode_attention_large_batch_block_split_context_traffic.json")) as f:
        d = json.load(f)
    assert 1.0 <= t / d["algorithmic_bytes_of_the_call"] <= 1.05
