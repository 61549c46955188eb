"""Plain, slow CPU oracle for the Block KV decode path (numpy, fp64).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library and imports
nothing from it; the two meet only on inputs drawn by the seeded generators.

Each function restates one passage of the pages in numpy, in the pages'
order, with no blocking, fusion or reordering beyond what the passage
states. Floating point is fp64; bf16 data is widened bit-exactly
(bf16 bits << 16 -> float32 -> float64).

Pages cited (by title):
  [BKV]  "Padding and Batching with Block KV" (AWS Neuron vllm-neuron docs)
  [BT]   "Block table: logical token -> physical KV block" (vLLM v0.25.1 notes)
  [KVC]  "KV Caching with vLLM" (AWS Neuron vllm-neuron docs)
  [CLB]  "Decode Context-Length Bucketing" (AWS Neuron vllm-neuron docs)

Where a page is silent the reading taken is stated at the function.
Every function here is pinned by CPU tests against values the pages print,
closed forms, library routines or brute force (tests/test_oracle_pins.py).
"""

from __future__ import annotations

import numpy as np

PAD_SLOT_ID = -1  # [BKV] "Slot ID -1: Padding Tokens"
NULL_BLOCK_ID = 0  # [BKV] "Block ID 0 vs. Sentinel -1"
P_MAX = 128  # [CLB] "Validation", rule 3


class OracleError(ValueError):
    """A rule of the pages rejects the input (carries a short code)."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


# ---------------------------------------------------------------------------
# Slot mapping
# ---------------------------------------------------------------------------
def compute_slot_mapping(req_indices, positions, block_table, block_size, max_num_tokens=None):
    """Slot id of every token; int64 array of length ``max_num_tokens``.

    Follows [BKV] "Slot Mapping Computation": a flat index
    ``req * max_blocks_per_req + pos // block_size`` into the raveled block
    table gives the physical block; the slot is that block times
    ``block_size`` plus ``pos % block_size`` ([BKV] "The Core Formula").
    Then the padding rules, in the order the pages apply them:

    * [BKV] "Slot Mapping for Padded Tokens": padding tokens are overwritten
      with -1. Reading: a padding token is one whose request index is -1
      (the caller marks them), or whose position is negative.
    * null block 0 and the -1 sentinel are never written ([BKV] "Block ID 0
      vs. Sentinel -1", "Slot ID -1"): a table entry <= 0 yields slot -1.
    * reading (the pages are silent): a position whose logical block lies
      past the table width, or a request index past the table's rows, yields
      slot -1.
    * [BT] data-flow listing: the last program pads the tail
      ``[num_tokens, max_num_tokens)`` with the pad id.
    """
    req = np.asarray(req_indices, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    table = np.asarray(block_table, dtype=np.int64)
    rows, max_blocks_per_req = table.shape
    num_tokens = len(req)
    if max_num_tokens is None:
        max_num_tokens = num_tokens
    assert max_num_tokens >= num_tokens and len(pos) == num_tokens

    # Which block in the table to look up (clamped only so the gather stays
    # inside the array; those tokens are overwritten just below).
    logical_block = np.where(pos >= 0, pos // block_size, 0)
    usable = (req >= 0) & (req < rows) & (pos >= 0) & (logical_block < max_blocks_per_req)
    block_table_indices = np.where(usable, req * max_blocks_per_req + logical_block, 0)
    block_numbers = table.ravel()[block_table_indices]
    block_offsets = np.where(pos >= 0, pos % block_size, 0)
    slot_mapping = block_numbers * block_size + block_offsets

    # Padding tokens and inactive blocks never write.
    slot_mapping = np.where(usable & (block_numbers > 0), slot_mapping, PAD_SLOT_ID)

    out = np.full(max_num_tokens, PAD_SLOT_ID, dtype=np.int64)
    out[:num_tokens] = slot_mapping
    return out


# ---------------------------------------------------------------------------
# Cache write
# ---------------------------------------------------------------------------
def reshape_and_cache(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Scatter each token's K/V rows into the paged caches, in place.

    Follows [BKV] "Slot ID -1: Padding Tokens": the write copies the new
    K (V) of token t to ``K_cache[slot_ids[t]]`` with out-of-bounds skip, so
    a slot of -1 (or any slot outside the cache) writes nothing.
    Caches are [total_blocks, block_size, Hkv, D] ([BKV] "Block Structure");
    one slot addresses one (block, offset) row of Hkv * D elements. The copy
    is of raw elements (storage dtype), so the result is a byte image.

    Reading: duplicate non-negative slots in one call are a caller error;
    this oracle rejects them.
    Returns the number of rows written.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    n_slots = nb * bs
    k_rows = k_cache.reshape(n_slots, *k_cache.shape[2:])
    v_rows = v_cache.reshape(n_slots, *v_cache.shape[2:])
    assert np.shares_memory(k_rows, k_cache) and np.shares_memory(v_rows, v_cache)
    T = k_new.shape[0]
    slots = slots[:T]
    # tokens whose slot lies inside the cache, and those slots
    live = np.nonzero((slots >= 0) & (slots < n_slots))[0]
    targets = slots[live]
    if np.unique(targets).size != targets.size:
        raise OracleError("duplicate_slot", "two tokens map to one slot")
    # one row copy per live token (targets are distinct, so order is immaterial)
    k_rows[targets] = k_new[live]
    v_rows[targets] = v_new[live]
    return int(live.size)


# ---------------------------------------------------------------------------
# Decode attention over the paged cache
# ---------------------------------------------------------------------------
def widen(x, dtype: str) -> np.ndarray:
    """Storage elements -> float64, exactly (bf16: bits << 16 is the float32)."""
    x = np.asarray(x)
    if dtype == "f32":
        return x.astype(np.float64)
    assert dtype == "bf16" and x.dtype == np.uint16
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, walk_blocks, scale,
                           dtype, requests=None, window=0, kv_pos_offset=None):
    """GQA decode attention over the paged cache, fp64; out [B, S_q, Hq, D].

    For request r with context length L = seq_lens[r] (the step's S_q new
    tokens already written), query token j sits at position L - S_q + j.
    Per [BKV] "Cache Masking", a query attends to cache positions below the
    cache length; the positions are absolute and independent of the table's
    values, so null or sentinel entries change nothing ([BKV] "Block ID 0 vs.
    Sentinel -1"). Readings:

    * the S_q tokens of one step attend causally among themselves (query j
      sees keys at positions <= its own); the page's all-ones active mask
      would let a draft see later drafts;
    * only the first ``walk_blocks`` table columns are visible: this is the
      head trim of [CLB] "Block-table head-trim vs. SWA tail-trim", which
      keeps logical blocks from 0 with absolute positions;
    * q head h uses KV head h // (Hq / Hkv) (consecutive groups, the
      "KV heads (after GQA)" of [BKV] "Block Structure");
    * a key whose table entry is <= 0 (inactive) contributes nothing;
    * a request with L <= 0 (a padded row) or a query with no visible key
      yields zeros.

    Sliding window ([KVC] "Attention Type": a sliding-window layer keeps only
    the recent tokens within the window; [CLB] "Block-table head-trim vs.
    SWA tail-trim"): with ``window`` > 0 the query at position qpos sees only
    keys at positions qpos - window + 1 .. qpos (the window counts the query's
    own position). With ``kv_pos_offset`` given, column c of request r's
    table row holds the block of absolute positions kv_pos_offset[r] + c * bs
    onward (the tail-trimmed frame; positions stay absolute); only positions
    from kv_pos_offset[r] up to kv_pos_offset[r] + walk_blocks * bs are
    visible.

    The key of position p is ``k_cache[block_table[r, (p - offset) // bs],
    p % bs, g]`` ([BKV] "Block Table"); scores are ``scale * <q, k>``; the
    output is the softmax-weighted sum of the values (max subtracted before
    exp). ``requests`` limits the computation to a subset of rows (others
    zero).
    """
    q64 = widen(q, dtype)
    B, S_q, Hq, D = q64.shape
    _, bs, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    assert G * Hkv == Hq
    table = np.asarray(block_table, dtype=np.int64)
    out = np.zeros((B, S_q, Hq, D), dtype=np.float64)
    rows = range(B) if requests is None else requests
    for r in rows:
        L = int(seq_lens[r])
        if L <= 0:
            continue
        off = 0 if kv_pos_offset is None else int(kv_pos_offset[r])
        assert off >= 0 and off % bs == 0
        visible_end = min(L, off + int(walk_blocks) * bs)
        positions = np.arange(off, max(visible_end, off))
        blocks = table[r, (positions - off) // bs]
        active = blocks > 0
        positions, blocks = positions[active], blocks[active]
        K = widen(k_cache[blocks, positions % bs], dtype)  # [n, Hkv, D]
        V = widen(v_cache[blocks, positions % bs], dtype)
        for j in range(S_q):
            qpos = L - S_q + j
            seen = positions <= qpos
            if window > 0:
                seen &= positions >= qpos - window + 1
            if not seen.any():
                continue
            Kj, Vj = K[seen], V[seen]
            for g in range(Hkv):
                # keys and values of KV head g, read by q heads g*G .. g*G + G - 1
                Kg = np.ascontiguousarray(Kj[:, g, :])
                Vg = np.ascontiguousarray(Vj[:, g, :])
                for h in range(g * G, (g + 1) * G):
                    s = scale * (Kg @ q64[r, j, h])
                    p = np.exp(s - s.max())
                    out[r, j, h] = (p @ Vg) / p.sum()
    return out


def swa_tail_trim(block_table, seq_lens, q_len, window, block_size):
    """Tail-trim a block table for a sliding-window layer; host only.

    [CLB] "Block-table head-trim vs. SWA tail-trim": a sliding-window layer
    keeps only the last blocks of each request and passes the position of
    the first kept block (swa_kv_pos_offset) so that positions stay
    absolute. Reading: the kept width is the number of blocks any window of
    this step can touch, ceil((window + q_len - 1) / bs) + 1 (the step's
    q_len queries need keys from L - q_len - window + 1 to L - 1, at any
    alignment; the page's window / block_size assumes one query and an
    aligned window), capped at the table width. Request r keeps the
    columns ending at its last context block (L - 1) // bs, starting no
    earlier than column 0; kept columns past the source table read -1.
    Returns (trimmed table [rows, width] int32, offsets [rows] int32).
    """
    t = np.asarray(block_table, dtype=np.int64)
    rows, src_w = t.shape
    width = min(src_w, -(-(window + q_len - 1) // block_size) + 1)
    out = np.full((rows, width), PAD_SLOT_ID, dtype=np.int64)
    offsets = np.zeros(rows, dtype=np.int64)
    for r in range(rows):
        L = int(seq_lens[r])
        last = (L - 1) // block_size if L > 0 else 0
        first = max(0, last - width + 1)
        offsets[r] = first * block_size
        for c in range(width):
            if first + c < src_w:
                out[r, c] = t[r, first + c]
    return out.astype(np.int32), offsets.astype(np.int32)


# ---------------------------------------------------------------------------
# Decode context parallelism (one rank's share)
# ---------------------------------------------------------------------------
def dcp_owner(position, world_size, interleave):
    """Rank that stores the KV of a position under decode context parallelism.

    [BT] design motivation ("DCP / PCP interleave"): with TOTAL_CP_WORLD_SIZE,
    TOTAL_CP_RANK and CP_KV_CACHE_INTERLEAVE_SIZE the slot-mapping kernel
    writes a real slot only for the positions its own rank stores and PAD_ID
    for the others. The page prints no formula. Reading: positions go to the
    ranks round-robin in runs of ``interleave`` consecutive tokens.
    """
    return (np.asarray(position) // interleave) % world_size


def dcp_local_position(position, world_size, interleave):
    """Position of a token inside its owner's cache (same reading).

    Each rank packs its own runs densely and in order: run k of the rank
    holds global runs k * world + rank. With ``interleave`` dividing the
    block size, the rank-local position's block index equals the global
    position // (world * block_size): every rank shares the request's table
    row, a table column standing for world * block_size consecutive
    positions (a "virtual" block), of which each rank stores block_size.
    """
    p = np.asarray(position)
    return (p // (world_size * interleave)) * interleave + p % interleave


def compute_slot_mapping_dcp(req_indices, positions, block_table, block_size, world_size, rank,
                             interleave, max_num_tokens=None):
    """Slot mapping on one context-parallel rank ([BT], as dcp_owner).

    A token this rank stores gets the slot of its rank-local position
    (table[r, lp // bs] * bs + lp % bs, with the padding, table-bounds and
    inactive-entry rules of compute_slot_mapping); every other token, and
    the tail of the buffer, gets PAD_SLOT_ID.
    """
    req = np.asarray(req_indices, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    assert block_size % interleave == 0 and 0 <= rank < world_size
    local = np.where(pos >= 0, dcp_local_position(np.maximum(pos, 0), world_size, interleave), -1)
    mine = (pos >= 0) & (dcp_owner(np.maximum(pos, 0), world_size, interleave) == rank)
    slots = compute_slot_mapping(req, local, block_table, block_size, max_num_tokens)
    n = len(req)
    slots[:n] = np.where(mine, slots[:n], PAD_SLOT_ID)
    return slots


def paged_decode_attention_dcp(q, k_cache, v_cache, block_table, seq_lens, walk_blocks, scale,
                               dtype, world_size, rank, interleave, requests=None):
    """One context-parallel rank's decode attention over the keys it stores.

    Queries are those of paged_decode_attention (global positions, causal);
    the keys are the positions p < L this rank owns (dcp_owner), read from
    this rank's cache at their rank-local position, with the head trim
    counted in table columns (p < walk_blocks * world * bs). Returns (out,
    lse): out normalised over this rank's keys, and the natural-log
    sum of exp(scores) over them (-inf and zeros where the rank sees no
    key), the partial state that ranks exchange and merge (merge_lse).
    """
    q64 = widen(q, dtype)
    B, S_q, Hq, D = q64.shape
    _, bs, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    assert block_size_ok(bs, interleave)
    table = np.asarray(block_table, dtype=np.int64)
    out = np.zeros((B, S_q, Hq, D), dtype=np.float64)
    lse = np.full((B, S_q, Hq), -np.inf, dtype=np.float64)
    rows = range(B) if requests is None else requests
    for r in rows:
        L = int(seq_lens[r])
        if L <= 0:
            continue
        visible = min(L, int(walk_blocks) * world_size * bs)
        gpos = np.arange(visible)
        gpos = gpos[dcp_owner(gpos, world_size, interleave) == rank]
        lpos = dcp_local_position(gpos, world_size, interleave)
        blocks = table[r, lpos // bs]
        active = blocks > 0
        gpos, lpos, blocks = gpos[active], lpos[active], blocks[active]
        K = widen(k_cache[blocks, lpos % bs], dtype)
        V = widen(v_cache[blocks, lpos % bs], dtype)
        for j in range(S_q):
            qpos = L - S_q + j
            seen = gpos <= qpos
            if not seen.any():
                continue
            Kj, Vj = K[seen], V[seen]
            for h in range(Hq):
                g = h // G
                s = scale * (Kj[:, g, :] @ q64[r, j, h])
                mx = s.max()
                p = np.exp(s - mx)
                out[r, j, h] = (p @ Vj[:, g, :]) / p.sum()
                lse[r, j, h] = mx + np.log(p.sum())
    return out, lse


def block_size_ok(block_size, interleave):
    """The reading of dcp_local_position needs the interleave to divide the block."""
    return interleave >= 1 and block_size % interleave == 0


def merge_lse(outs, lses):
    """Merge per-rank (out, lse) partial states into the full attention.

    The softmax over the union of the ranks' disjoint key sets: weight each
    rank's normalised output by exp(lse_rank - lse_total). Rows no rank saw
    stay zero.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    mx = lses.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - safe[None])  # exp(-inf) = 0 for ranks that saw nothing
    tot = w.sum(axis=0)
    merged = (w[..., None] * outs).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None]
    return np.where((tot > 0)[..., None], merged, 0.0)


# ---------------------------------------------------------------------------
# Context-length bucket selection
# ---------------------------------------------------------------------------
def smallest_bucket_at_least(n, buckets):
    """Smallest entry of ``buckets`` that is >= n, or None.

    The rule both bucket kinds use: [BKV] "Decode Batch Padding" (the
    scheduler picks the smallest batch bucket that fits) and [CLB]
    "Per-step bucket selection" (smallest bucket >= needed_seq).
    """
    fits = [b for b in buckets if b >= n]
    return min(fits) if fits else None


def select_batch_bucket(num_active, buckets):
    """Padded batch size of a decode step ([BKV] "Decode Batch Padding").

    The scheduler takes the smallest configured bucket that fits the active
    requests; the rows past them are dummy requests. Readings: the list
    must be non-empty, positive and strictly ascending (the page lists
    ascending buckets and states no rule; the context-bucket rules of [CLB]
    "Validation" minus its NKI tile rule), else code "bucket"; more active
    requests than the largest bucket is code "range" (the scheduler never
    schedules that many).
    """
    b = [int(x) for x in buckets]
    if not b or any(x <= 0 for x in b) or any(y <= x for x, y in zip(b, b[1:])):
        raise OracleError("bucket", "batch buckets must be positive and strictly ascending")
    if num_active < 0:
        raise OracleError("value", "negative request count")
    used = smallest_bucket_at_least(num_active, b)
    if used is None:
        raise OracleError("range", "more active requests than the largest batch bucket")
    return used


def validate_buckets(buckets, max_model_len):
    """[CLB] "Validation": a set list must be non-empty, positive, strictly
    ascending, each value below max_model_len and divisible by P_MAX = 128."""
    if len(buckets) == 0:
        raise OracleError("bucket", "empty list")
    for i, b in enumerate(buckets):
        if b <= 0:
            raise OracleError("bucket", f"non-positive {b}")
        if i and b <= buckets[i - 1]:
            raise OracleError("bucket", "not strictly ascending")
        if b >= max_model_len:
            raise OracleError("bucket", f"{b} not below max_model_len")
        if b % P_MAX:
            raise OracleError("bucket", f"{b} not divisible by {P_MAX}")


def select_ctx_bucket(max_num_computed_tokens, num_speculative_tokens, buckets, max_model_len,
                      block_size):
    """Per-step context bucket and the table columns it keeps.

    [CLB] "Per-step bucket selection": needed_seq = max(num_computed_tokens)
    + 1 + num_speculative_tokens; pick the smallest bucket >= needed_seq from
    the configured buckets plus max_model_len. [CLB] "Block-table head-trim":
    keep the first ceil(bucket / block_size) columns. [CLB] "Cross-DP
    synchronization" and "Backwards compatibility": with no buckets
    configured every step returns the full ceil(max_model_len / block_size).

    Readings: ``buckets`` None means unset (feature off); an empty list is
    a set list that fails validation; needed_seq beyond max_model_len is an
    error (the page skips the proposer rather than overflow the slots).
    Returns (bucket_len, walk_blocks).
    """
    if buckets is None:
        return max_model_len, -(-max_model_len // block_size)
    validate_buckets(list(buckets), max_model_len)
    needed_seq = max_num_computed_tokens + 1 + num_speculative_tokens
    if needed_seq > max_model_len:
        raise OracleError("range", f"needed_seq {needed_seq} > max_model_len {max_model_len}")
    bucket = smallest_bucket_at_least(needed_seq, list(buckets) + [max_model_len])
    return bucket, -(-bucket // block_size)


# ---------------------------------------------------------------------------
# Host-side table transforms
# ---------------------------------------------------------------------------
def remap_null_block_to_sentinel(block_table):
    """[BKV] "Block ID 0 vs. Sentinel -1": every 0 becomes -1."""
    t = np.asarray(block_table)
    return np.where(t == NULL_BLOCK_ID, -1, t).astype(t.dtype)


def map_to_kernel_blocks(block_table, manager_block_size, kernel_block_size):
    """Expand a manager-granularity table into kernel blocks.

    [BT] design motivation: one manager block becomes
    ``blocks_per_kv_block = manager / kernel`` kernel blocks, and a manager
    size the kernel size does not divide is rejected (ValueError). Reading
    of the unprinted formula, from the layout: a [N, bs, H, D] pool viewed
    as [N * k, bs / k, H, D] puts manager block m's i-th piece at kernel
    block m * k + i. Inactive entries (<= 0) stay inactive, k entries each,
    keeping their value.
    """
    if manager_block_size % kernel_block_size != 0:
        raise OracleError("value", "kernel block size must divide the manager block size")
    k = manager_block_size // kernel_block_size
    t = np.asarray(block_table, dtype=np.int64)
    rows, width = t.shape
    out = np.empty((rows, width * k), dtype=np.int64)
    for i in range(k):
        out[:, i::k] = np.where(t > 0, t * k + i, t)
    return out.astype(np.int32)


def kv_cache_tensor_bytes(num_blocks, block_size, num_kv_heads, head_size, element_bytes):
    """Bytes of one layer's K plus V pool ([KVC] KVCacheConfig example)."""
    return 2 * num_blocks * block_size * num_kv_heads * head_size * element_bytes
