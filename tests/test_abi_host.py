"""C-ABI checks that need no GPU.

The library loads and exports every function include/kvslot.h declares; the
host-only entry points (bucket selection, manager-to-kernel expansion) match
the oracle exactly; the GPU entry points reject bad scalars before any
device work (null pointers, so nothing could run even if the checks failed
open would crash rather than compute, and the calls return first).
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvslot.h")


@pytest.fixture(scope="module")
def K():
    import decode_attention_slot_amd as K

    if not os.path.exists(K.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    K.load()
    return K


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(K):
    names = declared_functions()
    assert len(names) >= 7
    assert set(names) == set(K.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(K.load(), n)


def test_status_strings(K):
    lib = K.load()
    for code in K.STATUS:
        assert lib.kvs_status_string(code).decode() != "unknown status"


def test_select_ctx_bucket_matches_oracle(K):
    configs = [([4096, 8192, 16384], 131072, 64), ([16384], 131072, 64), ([128, 512, 640], 1024, 16),
               (None, 131072, 64), (None, 1000, 64), ([128], 1000, 64)]
    rng = np.random.default_rng(0)
    for buckets, mml, bs in configs:
        ctxs = list(range(0, min(mml, 1100))) + list(rng.integers(0, mml + 10, size=300))
        for m in ctxs:
            for spec in (0, 1, 3):
                try:
                    want = O.select_ctx_bucket(int(m), spec, buckets, mml, bs)
                except O.OracleError as e:
                    with pytest.raises(K.KvslotError) as ke:
                        K.select_ctx_bucket(int(m), spec, buckets, mml, bs)
                    assert ke.value.name == {"range": "KVS_ERANGE", "bucket": "KVS_EBUCKET"}[e.code]
                    continue
                assert K.select_ctx_bucket(int(m), spec, buckets, mml, bs) == want


def test_select_ctx_bucket_validation_matches_oracle(K):
    import json

    g = json.load(open(os.path.join(ROOT, "tests", "golden", "clb_bucket_examples.json")))
    for bl in g["validation"]["invalid"]:
        with pytest.raises(K.KvslotError) as e:
            K.select_ctx_bucket(10, 0, bl, 131072, 64)
        assert e.value.name == "KVS_EBUCKET"
    for bl in g["validation"]["valid"]:
        K.select_ctx_bucket(10, 0, bl, 131072, 64)
    with pytest.raises(K.KvslotError) as e:
        K.select_ctx_bucket(-1, 0, [4096], 131072, 64)
    assert e.value.name == "KVS_EINVAL"


def test_select_batch_bucket_matches_oracle(K):
    lists = [[1, 2, 4, 8], [8], [1, 3, 5, 64, 256], [16, 32]]
    for b in lists:
        for n in range(0, max(b) + 3):
            try:
                want = ("ok", O.select_batch_bucket(n, b))
            except O.OracleError as e:
                want = (e.code, None)
            try:
                got = ("ok", K.select_batch_bucket(n, b))
            except K.KvslotError as e:
                got = ({"KVS_ERANGE": "range", "KVS_EBUCKET": "bucket"}[e.name], None)
            assert got == want, (b, n)
    for bad in ([], [0, 4], [4, 2], [2, 2]):
        with pytest.raises(K.KvslotError) as e:
            K.select_batch_bucket(1, bad)
        assert e.value.name == "KVS_EBUCKET"


def test_map_to_kernel_blocks_matches_oracle(K):
    rng = np.random.default_rng(3)
    for mgr_bs, kern_bs in ((32, 16), (64, 16), (16, 16), (256, 64)):
        t = rng.integers(-1, 5000, size=(9, 13)).astype(np.int32)
        assert np.array_equal(K.kv_map_to_kernel_blocks(t, mgr_bs, kern_bs),
                              O.map_to_kernel_blocks(t, mgr_bs, kern_bs))
    with pytest.raises(K.KvslotError):
        K.kv_map_to_kernel_blocks(np.ones((2, 2), np.int32), 32, 24)
    with pytest.raises(K.KvslotError):  # expanded id beyond int32
        K.kv_map_to_kernel_blocks(np.array([[2**30]], np.int32), 64, 16)


def test_gpu_entry_points_reject_bad_scalars(K):
    lib = K.load()
    null = None
    # kv_slot_mapping: negative sizes, max < num, bad stride / block size
    assert lib.kv_slot_mapping(null, null, -1, 0, null, 0, 1, 16, null, null) == -1
    assert lib.kv_slot_mapping(null, null, 5, 4, null, 0, 1, 16, null, null) == -1
    assert lib.kv_slot_mapping(null, null, 0, 0, null, 0, 0, 16, null, null) == -1
    assert lib.kv_slot_mapping(null, null, 0, 0, null, 0, 1, 0, null, null) == -1
    assert lib.kv_slot_mapping(null, null, 3, 3, null, 0, 1, 16, null, null) == -1  # null ptrs
    # kv_cache_write: bad dtype, row not a multiple of 16 bytes, null pointers
    assert lib.kv_cache_write(null, null, null, 1, null, null, 4, 16, 1, 64, 7, null) == -2
    assert lib.kv_cache_write(null, null, null, 1, null, null, 4, 16, 1, 2, 1, null) == -2
    assert lib.kv_cache_write(null, null, null, 1, null, null, 4, 16, 1, 64, 1, null) == -1
    assert lib.kv_cache_write(null, null, null, 0, null, null, 4, 16, 1, 64, 1, null) == 0

    # kv_slot_mapping_cache_write: the union of both checks
    def smw(T=1, M=1, rows=0, stride=1, bs=16, nb=4, hkv=1, d=64, dtype=1):
        return lib.kv_slot_mapping_cache_write(null, null, T, M, null, rows, stride, bs, null, null,
                                               null, null, null, nb, hkv, d, dtype, null)

    assert smw(T=-1) == -1 and smw(T=5, M=4) == -1 and smw(stride=0) == -1 and smw(bs=0) == -1
    assert smw(nb=0) == -1 and smw(hkv=0) == -1
    assert smw(dtype=7) == -2 and smw(d=2) == -2   # dtype; row of 4 bytes
    assert smw() == -1                             # null pointers
    assert smw(T=0, M=0) == 0                      # nothing to do

    def pda(**kw):
        a = dict(q=null, k=null, v=null, bt=null, stride=4, walk=4, sl=null, B=1, sq=1, hq=8, hkv=2,
                 d=128, bs=64, nb=10, scale=0.1, dtype=1, flags=0, ws=null, wsb=1 << 30, out=null)
        a.update(kw)
        return lib.paged_decode_attention(a["q"], a["k"], a["v"], a["bt"], a["stride"], a["walk"],
                                          a["sl"], a["B"], a["sq"], a["hq"], a["hkv"], a["d"], a["bs"],
                                          a["nb"], a["scale"], a["dtype"], a["flags"], a["ws"], a["wsb"],
                                          a["out"], null)

    assert pda() == -1                      # null pointers
    assert pda(B=0) == 0                    # nothing to do
    assert pda(hq=7) == -1                  # Hq not a multiple of Hkv
    assert pda(walk=5) == -1                # walk beyond the table
    assert pda(flags=2) == -1               # unknown flag
    assert pda(d=96) == -2                  # head_dim
    assert pda(bs=48) == -2                 # block size
    assert pda(bs=8) == -2
    assert pda(sq=17) == -2                 # 4 * 17 = 68 rows > 64
    assert pda(sq=16) == -1                 # 64 rows: supported (null pointers remain)
    assert pda(dtype=5) == -2
    assert pda(B=9000) == -2
    assert pda(scale=float("nan")) == -1
    assert lib.paged_decode_attention_workspace_bytes(1, 0, 8, 2, 128) == 0
    assert lib.paged_decode_attention_workspace_bytes(12, 1, 32, 8, 128) > 0


def test_swa_tail_trim_matches_oracle(K):
    rng = np.random.default_rng(5)
    for bs, q_len, window in [(16, 1, 1), (64, 4, 4096), (32, 2, 100), (256, 1, 5000), (16, 3, 17)]:
        lens = rng.integers(-3, 20000, size=11).astype(np.int32)
        lens[0], lens[1] = 0, 1
        width = int(-(-int(lens.max()) // bs)) + 3
        table = rng.integers(-1, 9999, size=(11, width)).astype(np.int32)
        got_t, got_o = K.kv_swa_tail_trim(table, lens, q_len, window, bs)
        want_t, want_o = O.swa_tail_trim(table, lens, q_len, window, bs)
        assert np.array_equal(got_t, want_t) and np.array_equal(got_o, want_o)


def test_swa_entry_points_reject_bad_scalars(K):
    lib = K.load()
    null = None
    import ctypes
    w = ctypes.c_int32()
    # kv_swa_tail_trim: bad window / q_len / block size, short destination, null pointers
    assert lib.kv_swa_tail_trim(null, 1, 4, null, 1, 0, 16, null, 4, null, ctypes.byref(w)) == -1
    assert lib.kv_swa_tail_trim(null, 1, 4, null, 0, 10, 16, null, 4, null, ctypes.byref(w)) == -1
    assert lib.kv_swa_tail_trim(null, 1, 40, null, 1, 100, 16, null, 2, null, ctypes.byref(w)) == -1
    assert w.value == 8  # ceil(100 / 16) + 1
    assert lib.kv_swa_tail_trim(null, 1, 40, null, 1, 100, 16, null, 8, null, ctypes.byref(w)) == -1
    assert lib.kv_swa_tail_trim(null, 0, 40, null, 1, 100, 16, null, 8, null, ctypes.byref(w)) == 0

    def swa(**kw):
        a = dict(q=null, k=null, v=null, bt=null, stride=4, walk=4, sl=null, off=null, win=8, B=1,
                 sq=1, hq=8, hkv=2, d=128, bs=64, nb=10, scale=0.1, dtype=1, ws=null,
                 wsb=1 << 30, out=null)
        a.update(kw)
        return lib.paged_decode_attention_swa(a["q"], a["k"], a["v"], a["bt"], a["stride"],
                                              a["walk"], a["sl"], a["off"], a["win"], a["B"],
                                              a["sq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
                                              a["scale"], a["dtype"], a["ws"], a["wsb"], a["out"],
                                              null)

    assert swa() == -1          # null pointers
    assert swa(win=-1) == -1    # negative window
    assert swa(B=0) == 0
    assert swa(d=96) == -2


def test_dcp_entry_points_reject_bad_scalars(K):
    lib = K.load()
    null = None

    def sm(world=2, rank=0, il=16, bs=64):
        return lib.kv_slot_mapping_dcp(null, null, 0, 0, null, 0, 1, bs, world, rank, il, null, null)

    assert sm() == 0
    assert sm(world=0) == -1 and sm(rank=2) == -1 and sm(rank=-1) == -1
    assert sm(il=3) == -1 and sm(il=128) == -1 and sm(il=0) == -1 and sm(bs=48) == -1

    def att(**kw):
        a = dict(B=1, world=2, rank=0, il=16, lse=null)
        a.update(kw)
        return lib.paged_decode_attention_dcp(null, null, null, null, 4, 4, null, a["B"], 1, 8, 2, 128,
                                              64, 10, 0.1, 1, a["world"], a["rank"], a["il"], null,
                                              1 << 30, null, a["lse"], null)

    assert att() == -1                # null lse / pointers
    assert att(B=0) == 0
    assert att(B=0, rank=3) == -1
    assert lib.decode_lse_merge(null, null, 0, 1, 128, null, null, null) == -1
    assert lib.decode_lse_merge(null, null, 2, 1, 6, null, null, null) == -1
    assert lib.decode_lse_merge(null, null, 2, 1, 128, null, null, null) == -1
    assert lib.decode_lse_merge(null, null, 2, 0, 128, null, null, null) == 0


def test_no_fallback_when_library_missing(K, tmp_path, monkeypatch):
    from decode_attention_slot_amd import _lib

    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.select_ctx_bucket(1, 0, None, 128, 16)
