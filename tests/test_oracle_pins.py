"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages print (fixtures under
tests/golden/, each with its citation), a closed form, a library routine, a
brute-force enumeration or an invariant the pages state. CPU only.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers (independent constructions; none calls the oracle)
# ---------------------------------------------------------------------------
def enumerate_slots(table, block_size):
    """(request, position) -> slot, by walking every table entry's offsets."""
    m = {}
    for r, row in enumerate(np.asarray(table)):
        for col, b in enumerate(row):
            if b > 0:
                for o in range(block_size):
                    m[(r, col * block_size + o)] = int(b) * block_size + o
    return m


def blockwise_cache(seqs, table, total_blocks, block_size, dtype):
    """Paged cache built block by block from logical sequences (no slots)."""
    Hkv, D = seqs[0].shape[1:]
    wl = W.Workload(name="", index=0, seed=0, dtype=dtype, block_size=block_size,
                    total_blocks=total_blocks, num_kv_heads=Hkv, num_q_heads=Hkv,
                    head_dim=D, q_len=1, num_reqs=0, computed=None, chunk_lens=None,
                    seq_lens=np.zeros(1), block_table=None)
    cache = wl.canary_cache()
    for r, seq in enumerate(seqs):
        for j in range(-(-len(seq) // block_size)):
            chunk = seq[j * block_size:(j + 1) * block_size]
            cache[table[r][j], :len(chunk)] = chunk
    return cache


def random_tables(rng, rows, width, lens, block_size, total_blocks, fill=-1):
    perm = rng.permutation(np.arange(1, total_blocks))
    table = np.full((rows, width), fill, np.int32)
    off = 0
    for r in range(rows):
        n = -(-int(lens[r]) // block_size)
        table[r, :n] = perm[off:off + n]
        off += n
    return table


def sdpa_reference(q64, K, V, L, S_q, scale, G, window=0):
    """torch's scaled_dot_product_attention (fp64, CPU) on contiguous keys.

    q64 [S_q, Hq, D]; K, V [n, Hkv, D] fp64 contiguous; query j sits at
    position L - S_q + j and sees keys at positions <= its own (and, with a
    window, above its own minus the window).
    """
    n = K.shape[0]
    qt = torch.from_numpy(q64).permute(1, 0, 2).unsqueeze(0)  # [1, Hq, S_q, D]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    qpos = torch.arange(S_q) + (L - S_q)
    mask = torch.arange(n)[None, :] <= qpos[:, None]  # [S_q, n]
    if window > 0:
        mask &= torch.arange(n)[None, :] > qpos[:, None] - window
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()  # [S_q, Hq, D]


# ---------------------------------------------------------------------------
# slot mapping
# ---------------------------------------------------------------------------
def test_slot_worked_examples():
    g = gold("bkv_slot_examples.json")
    for ex in g["examples"]:
        got = O.compute_slot_mapping(ex["req_indices"], ex["positions"],
                                     np.array(ex["block_table"], np.int32), ex["block_size"])
        assert got.tolist() == ex["expect_slots"], ex["cite"]


def test_slot_block_table_example():
    g = gold("bkv_slot_examples.json")["block_table_example"]
    table = np.array(g["block_table"], np.int32)
    for r, j, block in g["expect"]:
        # first and last token of logical block j land in physical block `block`
        s = O.compute_slot_mapping([r, r], [j * 64, j * 64 + 63], table, 64)
        assert s.tolist() == [block * 64, block * 64 + 63]


def test_prefill_with_padding():
    g = gold("bkv_slot_examples.json")["prefill_with_padding"]
    n, npad = g["actual_tokens"], g["padded_tokens"]
    table = np.array(g["block_table"], np.int32)
    req = np.array([0] * n + [-1] * (npad - n), np.int32)  # pads flagged by the caller
    pos = np.arange(npad, dtype=np.int64)
    slots = O.compute_slot_mapping(req, pos, table, g["block_size"])
    for t, s in g["expect_first_slots"].items():
        assert slots[int(t)] == s
    assert slots[:64].tolist() == list(range(640, 704))
    assert slots[64:100].tolist() == list(range(960, 996))
    assert (slots[n:] == g["expect_pad_slot"]).all()
    # the write: 100 actual writes, 28 skipped
    kc = np.zeros((16, 64, 1, 4), np.float32)
    vc = np.zeros_like(kc)
    knew = np.ones((npad, 1, 4), np.float32)
    written = O.reshape_and_cache(knew, knew, slots, kc, vc)
    assert written == g["expect_writes"]
    assert npad - written == g["expect_skipped"]


def test_decode_batch_padding():
    g = gold("bkv_slot_examples.json")["decode_batch_padding"]
    table = np.array([[3, 7, -1], [5, -1, -1]] + [[0, 0, 0]] * 6, np.int32)
    req = np.array([0, 1] + [-1] * 6, np.int32)
    pos = np.array([70, 20] + [0] * 6, np.int64)
    slots = O.compute_slot_mapping(req, pos, table, 64)
    assert slots.shape == (g["expect_shape"],)
    ref = enumerate_slots(table, 64)
    assert slots[:2].tolist() == [ref[(0, 70)], ref[(1, 20)]]
    assert (slots[g["active"]:] == g["expect_slot_tail"]).all()
    assert (pos[g["active"]:] == g["expect_positions_tail"]).all()


def test_multi_token_decode_count():
    g = gold("bkv_slot_examples.json")["multi_token_decode"]
    table = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9], [10, 11, 12]], np.int32)
    slots = O.compute_slot_mapping(g["req_indices"], g["positions"], table, 64)
    assert len(slots) == g["expect_total_tokens"]
    ref = enumerate_slots(table, 64)
    assert slots.tolist() == [ref[(r, p)] for r, p in zip(g["req_indices"], g["positions"])]


def test_slot_tail_padding():
    table = np.array([[4, 9]], np.int32)
    s = O.compute_slot_mapping([0, 0], [1, 70], table, 64, max_num_tokens=7)
    assert s.tolist() == [4 * 64 + 1, 9 * 64 + 6, -1, -1, -1, -1, -1]


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), bs=st.sampled_from([1, 2, 16, 32, 64]),
       rows=st.integers(1, 5), width=st.integers(1, 6))
def test_slot_brute_force(seed, bs, rows, width):
    rng = np.random.default_rng(seed)
    total = rows * width + 2
    ids = rng.permutation(np.arange(1, total))[: rows * width].reshape(rows, width)
    # sprinkle inactive entries: sentinel -1 and null block 0
    kill = rng.random((rows, width))
    table = np.where(kill < 0.2, -1, np.where(kill < 0.35, 0, ids)).astype(np.int32)
    T = 40
    req = rng.integers(-1, rows + 1, size=T).astype(np.int32)  # includes pads and a bad row
    pos = rng.integers(-2, (width + 1) * bs, size=T).astype(np.int64)  # includes past-width
    got = O.compute_slot_mapping(req, pos, table, bs, max_num_tokens=T + 3)
    ref = enumerate_slots(table, bs)
    want = [ref.get((int(r), int(p)), -1) if r >= 0 else -1 for r, p in zip(req, pos)] + [-1] * 3
    assert got.tolist() == want


def test_manager_kernel_expansion_layout():
    """map_to_kernel_blocks against a reshaped pool (numpy's own view)."""
    rng = np.random.default_rng(5)
    N, H, D = 9, 2, 3
    pool = rng.standard_normal((N, 32, H, D))
    kview = pool.reshape(N * 2, 16, H, D)  # the same memory at kernel granularity
    mgr = np.array([[3, 7, 1, -1], [8, 2, 0, 0]], np.int32)
    kt = O.map_to_kernel_blocks(mgr, 32, 16)
    assert kt.shape == (2, 8)
    for r in range(2):
        for c in range(4):
            m = mgr[r, c]
            for i in range(2):
                if m > 0:
                    np.testing.assert_array_equal(kview[kt[r, 2 * c + i]], pool[m, 16 * i:16 * i + 16])
                else:
                    assert kt[r, 2 * c + i] == m
    # and slots agree: the manager slot of every position equals the kernel slot
    req = np.repeat(np.arange(2), 128).astype(np.int32)
    pos = np.tile(np.arange(128), 2).astype(np.int64)
    np.testing.assert_array_equal(O.compute_slot_mapping(req, pos, mgr, 32),
                                  O.compute_slot_mapping(req, pos, kt, 16))


def test_manager_kernel_expansion_rejects_non_divisor():
    with pytest.raises(O.OracleError):
        O.map_to_kernel_blocks(np.ones((1, 2), np.int32), 32, 24)


def test_remap_null_block():
    t = np.array([[10, 15, 22, 0, 0], [8, 12, 0, 0, 0]], np.int32)
    assert O.remap_null_block_to_sentinel(t).tolist() == [[10, 15, 22, -1, -1], [8, 12, -1, -1, -1]]


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_write_matches_blockwise_image(dtype):
    rng = np.random.default_rng(11)
    bs, Hkv, D, total = 16, 2, 8, 24
    lens = [5, 33, 16]
    table = random_tables(rng, 3, 4, lens, bs, total)
    seqs = [W.to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in lens]
    want = blockwise_cache(seqs, table, total, bs, dtype)

    wl = W.Workload(name="", index=0, seed=0, dtype=dtype, block_size=bs, total_blocks=total,
                    num_kv_heads=Hkv, num_q_heads=Hkv, head_dim=D, q_len=1, num_reqs=0,
                    computed=None, chunk_lens=None, seq_lens=np.zeros(1), block_table=None)
    kc, vc = wl.canary_cache(), wl.canary_cache()
    req = np.concatenate([np.full(L, r, np.int32) for r, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    new = np.concatenate(seqs)
    # shuffle token order: the image must not depend on it
    order = rng.permutation(len(req))
    slots = O.compute_slot_mapping(req[order], pos[order], table, bs)
    n = O.reshape_and_cache(new[order], new[order], slots, kc, vc)
    assert n == sum(lens)
    assert kc.tobytes() == want.tobytes() and vc.tobytes() == want.tobytes()


def test_cache_write_skips_out_of_range_and_rejects_duplicates():
    kc = np.zeros((2, 4, 1, 2), np.float32)
    vc = np.zeros_like(kc)
    new = np.arange(8, dtype=np.float32).reshape(4, 1, 2)
    n = O.reshape_and_cache(new, new, [-1, 8, 100, 3], kc, vc)
    assert n == 1
    assert kc.reshape(8, 2)[3].tolist() == [6.0, 7.0]
    assert (np.delete(kc.reshape(8, 2), 3, axis=0) == 0).all()
    # slot 0 is inside the cache: only out-of-bounds slots are skipped
    n = O.reshape_and_cache(new[:1] + 1, new[:1] + 1, [0], kc, vc)
    assert n == 1 and kc.reshape(8, 2)[0].tolist() == [1.0, 2.0]
    with pytest.raises(O.OracleError):
        O.reshape_and_cache(new[:2], new[:2], [1, 1], kc, vc)


def test_kv_cache_tensor_size():
    g = gold("kvc_cache_config.json")
    got = O.kv_cache_tensor_bytes(g["num_blocks"], g["block_size"], g["num_kv_heads"],
                                  g["head_size"], g["element_bytes"])
    assert got == g["kv_cache_tensor_size"]


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def paged_case(rng, lens, bs, Hkv, G, D, S_q, dtype="f32", width=None, total=None):
    B = len(lens)
    width = width or max(-(-L // bs) for L in lens) + 1
    total = total or sum(-(-L // bs) for L in lens) + 3
    table = random_tables(rng, B, width, lens, bs, total)
    ks = [W.to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in lens]
    vs = [W.to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in lens]
    kc = blockwise_cache(ks, table, total, bs, dtype)
    vc = blockwise_cache(vs, table, total, bs, dtype)
    q = W.to_storage(rng.standard_normal((B, S_q, Hkv * G, D)).astype(np.float32), dtype)
    return dict(q=q, kc=kc, vc=vc, table=table, lens=np.array(lens, np.int32), ks=ks, vs=vs,
                width=width)


def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    c = paged_case(rng, [1, 1], bs=16, Hkv=2, G=2, D=8, S_q=1)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   0.3, "f32")
    for r in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[r, 0, h], c["vs"][r][0, h // 2].astype(np.float64))


def test_attention_zero_keys_average_values():
    rng = np.random.default_rng(2)
    c = paged_case(rng, [37], bs=16, Hkv=1, G=3, D=8, S_q=2)
    c["kc"][:] = 0
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   1.0, "f32")
    V = c["vs"][0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, 1], V[:36, 0].mean(axis=0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[0, 1, 2], V[:37, 0].mean(axis=0), rtol=0, atol=1e-12)


def test_attention_two_keys_closed_form():
    # scores 0 and ln 3 -> weights 1/4 and 3/4
    D, scale = 4, 0.5
    table = np.array([[1]], np.int32)
    kc = np.zeros((2, 2, 1, D), np.float32)
    vc = np.zeros_like(kc)
    kc[1, 1, 0, 0] = 1.0
    vc[1, 0, 0] = [1, 2, 3, 4]
    vc[1, 1, 0] = [5, 6, 7, 8]
    q = np.zeros((1, 1, 1, D), np.float32)
    q[0, 0, 0, 0] = np.float32(math.log(3.0) / scale)
    out = O.paged_decode_attention(q, kc, vc, table, np.array([2]), 1, scale, "f32")
    s1 = float(q[0, 0, 0, 0]) * scale  # the float32 q rounds ln 3 slightly
    w1 = math.exp(s1) / (1 + math.exp(s1))
    want = (1 - w1) * np.array([1, 2, 3, 4.0]) + w1 * np.array([5, 6, 7, 8.0])
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w1, 0.75, atol=1e-6)


def test_attention_dominant_key():
    rng = np.random.default_rng(3)
    c = paged_case(rng, [50], bs=16, Hkv=1, G=1, D=8, S_q=1)
    c["kc"][:] = 0
    b, o = c["table"][0, 20 // 16], 20 % 16
    c["q"][:] = 0
    c["q"][0, 0, 0, 0] = 1.0
    c["kc"][b, o, 0, 0] = 1000.0
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   1.0, "f32")
    np.testing.assert_allclose(out[0, 0, 0], c["vs"][0][20, 0], rtol=0, atol=1e-12)


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), bs=st.sampled_from([1, 2, 16, 64]),
       Hkv=st.sampled_from([1, 2]), G=st.sampled_from([1, 2, 4]), S_q=st.integers(1, 4),
       dtype=st.sampled_from(["f32", "bf16"]))
def test_attention_matches_sdpa_on_contiguous_keys(seed, bs, Hkv, G, S_q, dtype):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(S_q, 90, size=3)]
    D = 16
    c = paged_case(rng, lens, bs, Hkv, G, D, S_q, dtype)
    scale = 1 / math.sqrt(D)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   scale, dtype)
    for r, L in enumerate(lens):
        want = sdpa_reference(O.widen(c["q"][r], dtype), O.widen(c["ks"][r], dtype),
                              O.widen(c["vs"][r], dtype), L, S_q, scale, G)
        np.testing.assert_allclose(out[r], want, rtol=0, atol=1e-12)


def test_attention_head_trim_sees_only_walked_blocks():
    rng = np.random.default_rng(4)
    bs, D, G = 16, 8, 2
    c = paged_case(rng, [70], bs, 1, G, D, 1)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], 2, 0.4, "f32")
    want = sdpa_reference(O.widen(c["q"][0], "f32"), O.widen(c["ks"][0][:32], "f32"),
                          O.widen(c["vs"][0][:32], "f32"), 32, 1, 0.4, G)
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# sliding window and the SWA tail trim
# ---------------------------------------------------------------------------
def test_window_of_one_returns_each_querys_own_value():
    rng = np.random.default_rng(11)
    c = paged_case(rng, [40, 9], bs=16, Hkv=2, G=2, D=8, S_q=3)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   0.7, "f32", window=1)
    for r, L in enumerate([40, 9]):
        for j in range(3):
            for h in range(4):
                np.testing.assert_array_equal(out[r, j, h],
                                              c["vs"][r][L - 3 + j, h // 2].astype(np.float64))


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), bs=st.sampled_from([1, 16, 64]), G=st.sampled_from([1, 4]),
       S_q=st.integers(1, 4), window=st.integers(1, 120), dtype=st.sampled_from(["f32", "bf16"]))
def test_window_matches_sdpa_band_mask(seed, bs, G, S_q, window, dtype):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(S_q, 150, size=3)]
    D = 16
    c = paged_case(rng, lens, bs, 1, G, D, S_q, dtype)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                   0.25, dtype, window=window)
    for r, L in enumerate(lens):
        want = sdpa_reference(O.widen(c["q"][r], dtype), O.widen(c["ks"][r], dtype),
                              O.widen(c["vs"][r], dtype), L, S_q, 0.25, G, window=window)
        np.testing.assert_allclose(out[r], want, rtol=0, atol=1e-12)


def test_window_wider_than_context_is_full_attention():
    rng = np.random.default_rng(12)
    c = paged_case(rng, [33, 70], bs=16, Hkv=1, G=2, D=8, S_q=2)
    args = (c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"], 0.3, "f32")
    np.testing.assert_array_equal(O.paged_decode_attention(*args, window=70),
                                  O.paged_decode_attention(*args))


@pytest.mark.parametrize("seed", range(6))
def test_tail_trim_keeps_every_position_a_window_needs(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([16, 32, 64]))
    q_len, window = int(rng.integers(1, 5)), int(rng.integers(1, 300))
    lens = [int(x) for x in rng.integers(-2, 900, size=7)]
    src_w = max(-(-max(L, 1) // bs) for L in lens) + 2
    table = rng.permutation(np.arange(1, 7 * src_w + 1)).reshape(7, src_w).astype(np.int32)
    trimmed, off = O.swa_tail_trim(table, lens, q_len, window, bs)
    width = trimmed.shape[1]
    assert width == min(src_w, -(-(window + q_len - 1) // bs) + 1)
    for r, L in enumerate(lens):
        assert off[r] % bs == 0 and off[r] >= 0
        if L <= 0:
            continue
        assert (L - 1) // bs < off[r] // bs + width  # the last context block is kept
        for p in range(max(0, L - q_len - window + 1), L):  # every key any query sees
            assert p >= off[r]
            assert trimmed[r, (p - off[r]) // bs] == table[r, p // bs]


def test_tail_trimmed_frame_equals_full_table_with_window():
    rng = np.random.default_rng(13)
    lens, bs, S_q, window = [300, 17, 129, 64], 16, 2, 50
    c = paged_case(rng, lens, bs, 2, 2, 8, S_q)
    full = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"],
                                    0.3, "f32", window=window)
    trimmed, off = O.swa_tail_trim(c["table"], c["lens"], S_q, window, bs)
    got = O.paged_decode_attention(c["q"], c["kc"], c["vc"], trimmed, c["lens"], trimmed.shape[1],
                                   0.3, "f32", window=window, kv_pos_offset=off)
    np.testing.assert_array_equal(got, full)
    assert trimmed.shape[1] == 5 and off.tolist() == [224, 0, 64, 0]


# ---------------------------------------------------------------------------
# decode context parallelism: one rank's share
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("world,interleave,bs", [(1, 1, 16), (2, 1, 16), (2, 16, 16), (4, 8, 64),
                                                 (3, 4, 32), (8, 64, 64)])
def test_dcp_positions_partition_and_pack(world, interleave, bs):
    p = np.arange(0, 5 * world * bs + 7)
    owner = O.dcp_owner(p, world, interleave)
    local = O.dcp_local_position(p, world, interleave)
    assert set(owner.tolist()) <= set(range(world))
    for k in range(world):
        lp = local[owner == k]
        # each rank packs its own positions densely and in order
        assert lp.tolist() == list(range(len(lp)))
    # the rank-local block is the global "virtual" block of world * bs positions
    assert (local // bs == p // (world * bs)).all()
    # runs of interleave consecutive positions stay on one rank
    assert (owner == O.dcp_owner((p // interleave) * interleave, world, interleave)).all()


def test_dcp_slot_mapping_with_one_rank_is_plain():
    rng = np.random.default_rng(21)
    table = rng.permutation(np.arange(1, 41)).reshape(4, 10).astype(np.int32)
    table[1, 3] = -1
    req = rng.integers(-1, 5, size=300).astype(np.int32)
    pos = rng.integers(-2, 12 * 16, size=300)
    np.testing.assert_array_equal(O.compute_slot_mapping_dcp(req, pos, table, 16, 1, 0, 16, 333),
                                  O.compute_slot_mapping(req, pos, table, 16, 333))


def dcp_caches(rng, lens, bs, world, interleave, Hkv, D, dtype="f32"):
    """Every rank's cache, written through the DCP slot mapping of each rank."""
    B = len(lens)
    vblocks = [-(-L // (world * bs)) for L in lens]
    width = max(vblocks) + 1
    total = sum(vblocks) + 2
    table = random_tables(rng, B, width, [n * bs for n in vblocks], bs, total)
    ks = [W.to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in lens]
    vs = [W.to_storage(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype) for L in lens]
    req = np.concatenate([np.full(L, r, np.int32) for r, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L) for L in lens])
    knew, vnew = np.concatenate(ks), np.concatenate(vs)
    wl = W.Workload(name="", index=0, seed=0, dtype=dtype, block_size=bs, total_blocks=total,
                    num_kv_heads=Hkv, num_q_heads=Hkv, head_dim=D, q_len=1, num_reqs=0,
                    computed=None, chunk_lens=None, seq_lens=np.zeros(1), block_table=None)
    caches = []
    for k in range(world):
        slots = O.compute_slot_mapping_dcp(req, pos, table, bs, world, k, interleave)
        kc, vc = wl.canary_cache(), wl.canary_cache()
        O.reshape_and_cache(knew, vnew, slots, kc, vc)
        caches.append((kc, vc, slots))
    return table, ks, vs, caches, width


@pytest.mark.parametrize("world,interleave", [(2, 1), (2, 16), (4, 8), (3, 16)])
def test_dcp_every_token_stored_once_and_found(world, interleave):
    rng = np.random.default_rng(22)
    lens, bs = [1, 40, 200], 16
    table, ks, _, caches, _ = dcp_caches(rng, lens, bs, world, interleave, 2, 4)
    stored = sum((c[2] >= 0).sum() for c in caches)
    assert stored == sum(lens)
    for r, L in enumerate(lens):
        for p in range(L):
            k = int(O.dcp_owner(p, world, interleave))
            lp = int(O.dcp_local_position(p, world, interleave))
            row = caches[k][0][table[r, lp // bs], lp % bs]
            np.testing.assert_array_equal(row, ks[r][p])


@pytest.mark.parametrize("world,interleave,S_q", [(2, 1, 1), (2, 16, 3), (4, 8, 2), (3, 4, 1)])
def test_dcp_merged_ranks_equal_full_attention(world, interleave, S_q):
    rng = np.random.default_rng(23)
    lens, bs, Hkv, G, D = [S_q, 37, 150, 301], 16, 2, 2, 8
    table, ks, vs, caches, width = dcp_caches(rng, lens, bs, world, interleave, Hkv, D)
    q = rng.standard_normal((len(lens), S_q, Hkv * G, D)).astype(np.float32)
    parts = [O.paged_decode_attention_dcp(q, kc, vc, table, np.array(lens), width, 0.35, "f32",
                                          world, k, interleave)
             for k, (kc, vc, _) in enumerate(caches)]
    merged = O.merge_lse([o for o, _ in parts], [l for _, l in parts])
    for r, L in enumerate(lens):
        want = sdpa_reference(O.widen(q[r], "f32"), O.widen(ks[r], "f32"), O.widen(vs[r], "f32"),
                              L, S_q, 0.35, G)
        np.testing.assert_allclose(merged[r], want, rtol=0, atol=1e-12)


def test_dcp_lse_of_a_single_key_is_its_score():
    rng = np.random.default_rng(24)
    table, ks, _, caches, width = dcp_caches(rng, [1], 16, 2, 1, 1, 4)
    q = rng.standard_normal((1, 1, 1, 4)).astype(np.float32)
    out, lse = O.paged_decode_attention_dcp(q, caches[0][0], caches[0][1], table, np.array([1]),
                                            width, 0.5, "f32", 2, 0, 1)
    score = 0.5 * float(ks[0][0, 0].astype(np.float64) @ q[0, 0, 0].astype(np.float64))
    assert abs(lse[0, 0, 0] - score) < 1e-12
    _, lse1 = O.paged_decode_attention_dcp(q, caches[1][0], caches[1][1], table, np.array([1]),
                                           width, 0.5, "f32", 2, 1, 1)
    assert lse1[0, 0, 0] == -np.inf  # rank 1 stores nothing of a 1-token request


def test_bf16_widening_matches_torch():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x4049, 0xC2F7], np.uint16)
    rng = np.random.default_rng(0)
    bits = np.concatenate([bits, rng.integers(0, 0x7F80, size=200).astype(np.uint16)])
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.widen(bits, "bf16"), want)


def test_invariant_sentinel_vs_null_block():
    """Null block 0 vs sentinel -1 in unused entries: identical output."""
    rng = np.random.default_rng(6)
    c = paged_case(rng, [20, 45, 3], 16, 2, 2, 8, 2)
    t0 = np.where(c["table"] < 0, 0, c["table"])
    tm = O.remap_null_block_to_sentinel(t0)
    a = O.paged_decode_attention(c["q"], c["kc"], c["vc"], t0, c["lens"], c["width"], 0.3, "f32")
    b = O.paged_decode_attention(c["q"], c["kc"], c["vc"], tm, c["lens"], c["width"], 0.3, "f32")
    assert a.tobytes() == b.tobytes()


def test_invariant_bucketed_equals_full_walk():
    rng = np.random.default_rng(7)
    c = paged_case(rng, [20, 45, 3], 16, 2, 2, 8, 1, width=40)
    full = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], 40, 0.3, "f32")
    trim = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], 3, 0.3, "f32")
    assert full.tobytes() == trim.tobytes()


def test_invariant_physical_block_relabelling():
    rng = np.random.default_rng(8)
    c = paged_case(rng, [20, 45, 33], 16, 2, 2, 8, 3)
    total = c["kc"].shape[0]
    relabel = np.concatenate([[0], rng.permutation(np.arange(1, total))])
    kc2, vc2 = np.empty_like(c["kc"]), np.empty_like(c["vc"])
    kc2[relabel], vc2[relabel] = c["kc"], c["vc"]
    t2 = np.where(c["table"] > 0, relabel[np.maximum(c["table"], 0)], c["table"])
    a = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"], 0.3, "f32")
    b = O.paged_decode_attention(c["q"], kc2, vc2, t2, c["lens"], c["width"], 0.3, "f32")
    assert a.tobytes() == b.tobytes()


def test_invariant_causality():
    """Changing K/V after a query's position leaves that query's output alone."""
    rng = np.random.default_rng(9)
    bs, S_q = 16, 4
    c = paged_case(rng, [40], bs, 1, 2, 8, S_q)
    a = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], c["lens"], c["width"], 0.3, "f32")
    p = 38  # query 2 sits at 38, query 3 at 39
    b_, o_ = c["table"][0, p // bs], p % bs
    kc2, vc2 = c["kc"].copy(), c["vc"].copy()
    kc2[b_, o_ + 1] += 5.0
    vc2[b_, o_ + 1] -= 3.0
    b = O.paged_decode_attention(c["q"], kc2, vc2, c["table"], c["lens"], c["width"], 0.3, "f32")
    assert a[0, :3].tobytes() == b[0, :3].tobytes()
    assert not np.allclose(a[0, 3], b[0, 3])


@pytest.mark.parametrize("hole", [-1, 0])
def test_inactive_entry_inside_context_contributes_nothing(hole):
    rng = np.random.default_rng(12)
    bs, D, G = 16, 8, 2
    c = paged_case(rng, [40], bs, 1, G, D, 1)
    t = c["table"].copy()
    t[0, 1] = hole  # keys 16..31 lose their block
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], t, c["lens"], c["width"], 0.4, "f32")
    keep = np.r_[0:16, 32:40]
    want = sdpa_reference(O.widen(c["q"][0], "f32"), O.widen(c["ks"][0][keep], "f32"),
                          O.widen(c["vs"][0][keep], "f32"), len(keep), 1, 0.4, G)
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)


def test_padded_rows_yield_zero():
    rng = np.random.default_rng(10)
    c = paged_case(rng, [20, 1], 16, 1, 2, 8, 1)
    lens = np.array([20, 0], np.int32)
    out = O.paged_decode_attention(c["q"], c["kc"], c["vc"], c["table"], lens, c["width"], 0.3, "f32")
    assert (out[1] == 0).all() and np.abs(out[0]).sum() > 0


# ---------------------------------------------------------------------------
# context-length bucket selection
# ---------------------------------------------------------------------------
def test_bucket_examples_from_the_page():
    g = gold("clb_bucket_examples.json")
    for part in ("single_bucket", "multi_bucket", "needed_seq"):
        ex = g[part]
        for max_ctx, spec, want in ex["cases"]:
            b, walk = O.select_ctx_bucket(max_ctx, spec, ex["buckets"], ex["max_model_len"],
                                          ex["block_size"])
            assert b == want, (part, max_ctx, spec)
            assert walk == -(-want // ex["block_size"])


def test_head_trim_block_counts():
    for bucket, bs, want in gold("clb_bucket_examples.json")["head_trim"]["cases"]:
        buckets = [b for b in (4096, 8192, 16384) if b <= bucket and b < 131072]
        _, walk = O.select_ctx_bucket(bucket - 1, 0, buckets or None, 131072, bs)
        assert walk == want


def test_full_walk_rounds_up():
    for mml, bs, want in gold("clb_bucket_examples.json")["full_ceil"]["cases"]:
        assert O.select_ctx_bucket(0, 0, None, mml, bs) == (mml, want)
        # the max_model_len fallback of a configured list rounds up the same way
        assert O.select_ctx_bucket(mml - 1, 0, [128], mml, bs) == (mml, want)


def test_feature_off_returns_full():
    g = gold("clb_bucket_examples.json")["full_when_unset"]
    for max_ctx in (0, 100, 5000, 131000):
        assert O.select_ctx_bucket(max_ctx, 3, None, g["max_model_len"], g["block_size"]) == (
            g["expect_bucket"], g["expect_walk_blocks"])


def test_bucket_validation():
    g = gold("clb_bucket_examples.json")["validation"]
    for bl in g["valid"]:
        O.validate_buckets(bl, g["max_model_len"])
    for bl in g["invalid"]:
        with pytest.raises(O.OracleError) as e:
            O.select_ctx_bucket(10, 0, bl, g["max_model_len"], 64)
        assert e.value.code == "bucket"


def test_needed_seq_beyond_max_model_len():
    with pytest.raises(O.OracleError) as e:
        O.select_ctx_bucket(131071, 1, [4096], 131072, 64)
    assert e.value.code == "range"
    assert O.select_ctx_bucket(131071, 0, [4096], 131072, 64) == (131072, 2048)


def test_amplification_ratio():
    g = gold("clb_bucket_examples.json")["amplification"]
    _, full = O.select_ctx_bucket(g["effective_kv"] - 1, 0, None, g["max_model_len"], 64)
    _, trim = O.select_ctx_bucket(g["effective_kv"] - 1, 0, [4096], g["max_model_len"], 64)
    assert full // trim == g["ratio"]


def test_bucket_cover_minimal_monotone_and_dp_agreement():
    buckets, mml, bs = [128, 512, 640], 1024, 16
    prev = 0
    for max_ctx in range(0, mml):
        for spec in range(0, 4):
            needed = max_ctx + 1 + spec
            if needed > mml:
                continue
            b, walk = O.select_ctx_bucket(max_ctx, spec, buckets, mml, bs)
            cands = buckets + [mml]
            assert b in cands and b >= needed  # covers every KV the step touches
            assert not [c for c in cands if needed <= c < b]  # smallest such
            assert walk * bs >= b > (walk - 1) * bs
        b0, _ = O.select_ctx_bucket(max_ctx, 0, buckets, mml, bs)
        assert b0 >= prev  # monotone in max_ctx
        prev = b0
    # ranks agree by taking the max over ranks; the agreed pick covers every
    # rank's own need, and idle ranks contributing 0 change nothing
    rng = np.random.default_rng(0)
    for _ in range(50):
        busy = [int(x) for x in rng.integers(0, mml - 4, size=4)]
        agreed = max(busy + [0, 0])
        pick = O.select_ctx_bucket(agreed, 3, buckets, mml, bs)
        assert pick == O.select_ctx_bucket(max(busy), 3, buckets, mml, bs)
        for m in busy:
            assert pick[0] >= O.select_ctx_bucket(m, 3, buckets, mml, bs)[0]


def test_num_seqs_bucket_table():
    g = gold("bkv_num_seqs_buckets.json")
    for active, used, pad in g["rows"]:
        assert O.smallest_bucket_at_least(active, g["buckets"]) == used
        assert used - active == pad
    s = g["single_bucket"]
    assert O.smallest_bucket_at_least(s["active"], s["buckets"]) == s["bucket_used"]


def test_batch_bucket_selection_follows_the_page():
    g = gold("bkv_num_seqs_buckets.json")
    for active, used, pad in g["rows"]:
        assert O.select_batch_bucket(active, g["buckets"]) == used
    s = g["single_bucket"]
    for active in range(1, 9):  # a single bucket of 8 serves every batch size
        assert O.select_batch_bucket(active, s["buckets"]) == s["bucket_used"]
    for bad in ([], [0, 4], [4, 2], [2, 2]):
        with pytest.raises(O.OracleError) as e:
            O.select_batch_bucket(1, bad)
        assert e.value.code == "bucket"
    with pytest.raises(O.OracleError) as e:
        O.select_batch_bucket(9, g["buckets"])
    assert e.value.code == "range"
