"""Benchmark of the Block KV decode step on one MI355X.

One step = the whole hot path over one batch: the host bucket pick
(select_ctx_bucket), then on the GPU the slot mapping and cache write of the
step's new tokens and the decode attention. By default the GPU part is one
paged_decode_attention_append call (the decode launch writes the step's rows
itself when they qualify); --fused-write runs kv_slot_mapping_cache_write
then paged_decode_attention, --separate-write kv_slot_mapping and
kv_cache_write then paged_decode_attention. Inputs are seeded and synthetic
and already resident in HBM when the timed region starts (the prior context
is prefilled through the library beforehand, untimed). The default workload
is the largest single-GPU one: 256 decode requests (+8 padded rows) over a
kernel block size of 16, GQA 8, about 4.5 GB of KV per step.

Timing: the K timed steps run back to back, bracketed by synchronisations,
and give the wall time per step. After them, the step's attention call (with
the append, the call that also writes the step's rows) runs --calls more
times (100 by default, never fewer than 50, whatever --steps says), each call
bracketed by its own pair of HIP events; the median of those durations is the
roofline figure. The events are created with hipEventDisableSystemFence: a
default event's record also writes back and invalidates the caches at system
scope, which adds to the timed work. The slot mapping and cache write kernels
and their one-launch fusion are timed after that, each in a run of
back-to-back launches.

The step rotates over several identical copies of the KV cache when one
step's bytes are below 1 GiB, so that the bytes a step reads come from HBM,
not from the last step's L2 / MALL lines.

Prints one JSON line: whole-step throughput (algorithmic bytes of every
kernel / wall time per step), decode and slot-mapping tokens/s, a roofline
entry for the attention call (algorithmic bytes / its event-timed median
duration against 8 TB/s) and the CPU oracle timed on a bounded sample, on
one host core and on all the host cores the process may use.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MIN_CALLS = 50  # event-timed attention calls, at least
SLOT_SWEEP_TOKENS = 1 << 22  # slot mapping measured at this many tokens per launch as well
SLOT_SWEEP_SETS = 11  # distinct token sets rotated (11 x 100 MB: past the 256 MB MALL)
SLOT_SWEEP_RUN = 128  # consecutive positions per request in the chunked sweep
WORKLOADS = {
    "block_config_bf16": 1,
    "ctx_bucketing": 2,
    "large_batch_block_split": 3,
    "ragged_spec_decode": 4,
    "tiny_fp32": 0,
}
DESCRIPTIONS = {
    0: "tiny fp32: 2 requests (ctx 3, 100), bs 64, Hkv 2, Hq 8, D 64",
    1: "block config bf16: 12 decode requests, ctx U[1,5000], 1024 blocks of 64, Hkv 8, Hq 32, D 128",
    2: "context-length bucketing bf16: 8 requests, lognormal ctx (median 4096), max_model_len 131072, "
       "buckets [4096, 8192, 16384], bs 64, Hkv 8, Hq 32, D 128",
    3: "large batch bf16: 256 requests (+8 padded rows), ctx U[512,8192], manager bs 32 split to "
       "kernel bs 16, Hkv 8, Hq 64, D 128",
    "3spec": "large batch bf16 with speculative decode: 256 requests (+8 padded rows), ctx "
             "U[512,8192], 1+{n} causal decode tokens each, manager bs 32 split to kernel bs 16, "
             "Hkv 8, Hq 64, D 128",
    4: "ragged + speculative bf16: 64 requests, 8192-token ragged chunk, then 1+3 causal decode "
       "tokens each, bs 64, Hkv 8, Hq 32, D 128",
}
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_slot_amd", "csrc", f)
                  for f in ("paged_decode.h", "paged_decode.hip", "paged_decode_nc2.hip",
                            "paged_decode_nc4.hip")]


def kernel_source_hash() -> str:
    """sha256[:16] of the decode kernels' code: the sources with // comments,
    trailing blanks and empty lines removed, so that editing a comment does not
    retire a counter measurement of unchanged code."""
    lines = []
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


class HipEvent:
    """A HIP timing event recorded on a given stream, created with
    hipEventDisableSystemFence: recording it writes a timestamp without the
    system-scope cache writeback and invalidation a default event performs,
    which would otherwise add to (and perturb) the work being timed. Uses the
    HIP runtime the process already runs (torch's, which the library shares).
    """

    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            import ctypes

            import torch

            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self._ev = ctypes.c_void_p()
        if self._rt().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream_ptr: int) -> None:
        if self._rt().hipEventRecord(self._ev, stream_ptr):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        import ctypes

        ms = ctypes.c_float()
        if self._rt().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


def attention_bytes(w, walk_blocks: int, table_walk: bool) -> int:
    """Algorithmic bytes of one attention launch (whole blocks, the DMA unit).

    Per request: the KV blocks it must read (context blocks, or every walked
    column in the fixed-shape walk) at 2 * bs * Hkv * D * es bytes each plus
    a 4-byte table entry; q in the cache dtype, fp32 out, and its seq_len.
    """
    es = w.es
    per_block = 2 * w.block_size * w.num_kv_heads * w.head_dim * es + 4
    blocks = 0
    for r in range(w.num_rows):
        L = int(w.seq_lens[r])
        vis = min(max(L, 0), walk_blocks * w.block_size)
        blocks += walk_blocks if table_walk else -(-vis // w.block_size)
    q_out = w.num_rows * w.q_len * w.num_q_heads * w.head_dim * (es + 4)
    return blocks * per_block + q_out + 4 * w.num_rows


def attention_bytes_token_exact(w, walk_blocks: int) -> int:
    """Lower bound beside the block count: only the K and V rows of the
    visible positions (L instead of whole blocks), one table entry per block
    holding one, q, fp32 out and seq_len."""
    es = w.es
    per_token = 2 * w.num_kv_heads * w.head_dim * es
    total = 0
    for r in range(w.num_rows):
        vis = min(max(int(w.seq_lens[r]), 0), walk_blocks * w.block_size)
        total += vis * per_token + 4 * (-(-vis // w.block_size))
    q_out = w.num_rows * w.q_len * w.num_q_heads * w.head_dim * (es + 4)
    return total + q_out + 4 * w.num_rows


def dcp_attention_bytes(w, world: int, rank: int, interleave: int) -> int:
    """Algorithmic bytes of one rank's decode attention under context parallelism.

    Per request: the whole blocks of this rank's cache holding its share of
    the context (the positions below L it stores, packed densely), plus a
    table entry each; q in; fp32 out and lse; seq_len.
    """
    per_block = 2 * w.block_size * w.num_kv_heads * w.head_dim * w.es + 4
    span = world * interleave
    blocks = 0
    for r in range(w.num_rows):
        L = int(w.seq_lens[r])
        if L <= 0:
            continue
        local = (L // span) * interleave + min(max(L % span - rank * interleave, 0), interleave)
        blocks += -(-local // w.block_size)
    rows = w.num_rows * w.q_len * w.num_q_heads
    return blocks * per_block + rows * w.head_dim * (w.es + 4) + 4 * rows + 4 * w.num_rows


def window_attention_bytes(w, window: int, kv_off, width: int) -> int:
    """Algorithmic bytes of one sliding-window launch over a tail-trimmed table.

    Per request: the whole blocks holding the keys some query of the step
    sees (positions L - S_q - window + 1 .. L - 1, within the trimmed
    columns), plus a table entry each; q in, fp32 out, seq_len and offset.
    """
    per_block = 2 * w.block_size * w.num_kv_heads * w.head_dim * w.es + 4
    bs = w.block_size
    blocks = 0
    for r in range(w.num_rows):
        L = int(w.seq_lens[r])
        if L <= 0:
            continue
        off = int(kv_off[r])
        end = min(L, off + width * bs)
        start = max(off, L - w.q_len - window + 1)
        if end > start:
            blocks += -(-end // bs) - start // bs
    q_out = w.num_rows * w.q_len * w.num_q_heads * w.head_dim * (w.es + 4)
    return blocks * per_block + q_out + 8 * w.num_rows


def slot_map_bytes(T: int) -> int:
    """24 bytes per token: request index, position, table entry, slot."""
    return 24 * T


def cache_write_bytes(w, T_live: int, T: int) -> int:
    """Each written token reads and writes its K and V rows; every slot is read."""
    row = w.num_kv_heads * w.head_dim * w.es
    return T_live * 4 * row + 8 * T


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="large_batch_block_split", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--walk", default="context", choices=["context", "bucket", "full"],
                    help="context: read only covering blocks; bucket/full: fixed-shape walk of the "
                         "bucket's or the whole table's columns")
    ap.add_argument("--max-ctx", type=int, default=None,
                    help="bucketing workload: clip the drawn context lengths and pin the largest")
    ap.add_argument("--num-spec", type=int, default=0,
                    help="large-batch workload: decode 1 + this many causal tokens per request "
                         "(3: 32 query rows per KV head)")
    ap.add_argument("--rotate", type=int, default=0, help="cache copies to rotate over (0 = auto)")
    ap.add_argument("--calls", type=int, default=100,
                    help="event-timed attention calls after the steps (median; at least 50)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time per leg (one core, then every core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window layer: attend over a tail-trimmed table with this window "
                         "(paged_decode_attention_swa); the trim is host metadata built untimed")
    ap.add_argument("--batch-buckets", default=None,
                    help="comma-separated num_seqs buckets: pad the batch with dummy requests to the "
                         "smallest that fits (select_batch_bucket, called every step)")
    ap.add_argument("--dcp", type=int, default=1,
                    help="decode context parallelism over this many ranks: measure rank 0's share "
                         "(its cache holds only its tokens; paged_decode_attention_dcp)")
    ap.add_argument("--dcp-interleave", type=int, default=1)
    ap.add_argument("--tp", type=int, default=1,
                    help="tensor parallelism over KV heads: measure one rank's share "
                         "(num_kv_heads / tp KV heads and the matching query heads)")
    ap.add_argument("--separate-write", action="store_true",
                    help="step uses kv_slot_mapping + kv_cache_write (two launches), then "
                         "paged_decode_attention")
    ap.add_argument("--fused-write", action="store_true",
                    help="step uses kv_slot_mapping_cache_write, then paged_decode_attention, "
                         "instead of paged_decode_attention_append")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the steps, run one plain device copy of this size (counter scale)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the "
              "sharding design is per-GPU and exchange-free); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import decode_attention_slot_amd as K
    import workloads as W
    from workloads import device as dev

    if not os.path.exists(K.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    lib = K.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cuda = torch.device("cuda:0")
    idx = WORKLOADS[args.workload]
    extra = {"forced_max_ctx": args.max_ctx} if (idx == 2 and args.max_ctx is not None) else {}
    if args.num_spec:
        if idx != 3:
            raise SystemExit("--num-spec applies to the large-batch workload")
        extra["num_spec"] = args.num_spec
    w = W.make_workload(idx, seed=args.seed, **extra)
    if args.tp > 1:
        w = W.tp_share(w, args.tp)
    batch_buckets = [int(x) for x in args.batch_buckets.split(",")] if args.batch_buckets else None
    num_active = w.num_rows
    if batch_buckets:
        w = W.pad_batch(w, K.select_batch_bucket(num_active, batch_buckets))

    # ---- set-up (untimed): caches, prefill, rotation copies ---------------
    t_setup = time.time()
    dcp = (args.dcp, 0, args.dcp_interleave) if args.dcp > 1 else None
    if dcp and (args.window or args.walk != "context"):
        raise SystemExit("--dcp takes the context walk without a window")
    s = dev.build(w, cuda, threads=16, dcp=dcp)
    table_walk = args.walk != "context"
    # tokens each request holds before its decode tokens (prior context + ragged chunk)
    before = (w.computed + w.chunk_lens)[: w.num_reqs]
    max_ctx = int(before.max()) if w.num_reqs else 0
    num_spec = w.q_len - 1
    buckets = w.buckets if args.walk == "bucket" else None
    max_model_len = w.table_width * w.block_size
    bucket_len, walk_blocks = K.select_ctx_bucket(max_ctx, num_spec, buckets, max_model_len,
                                                  w.block_size)
    walk_blocks = min(walk_blocks, w.table_width)

    step_req = torch.cat([s.chunk_req, s.dec_req]).contiguous()
    step_pos = torch.cat([s.chunk_pos, s.dec_pos]).contiguous()
    step_k = torch.cat([s.chunk_k, s.dec_k]).contiguous()
    step_v = torch.cat([s.chunk_v, s.dec_v]).contiguous()
    T = int(step_req.numel())
    T_live = int((step_req >= 0).sum().item())
    a_bytes = attention_bytes(w, walk_blocks, table_walk)
    exact_bytes = attention_bytes_token_exact(w, walk_blocks)
    if dcp or args.window:
        exact_bytes = None  # reported for the plain walks only
    if dcp:
        a_bytes = dcp_attention_bytes(w, *dcp)
        walk_blocks = int(s.block_table.shape[1])
    if args.window:
        if table_walk:
            raise SystemExit("--window takes the context walk")
        lens_h = w.seq_lens[: w.num_rows].astype(np.int32)
        trimmed, kv_off = K.kv_swa_tail_trim(s.host_table, lens_h, w.q_len, args.window,
                                             w.block_size)
        d_trim = torch.from_numpy(trimmed).to(cuda)
        d_off = torch.from_numpy(kv_off).to(cuda)
        a_bytes = window_attention_bytes(w, args.window, kv_off, trimmed.shape[1])
    kv_bytes_touched = a_bytes
    if args.rotate > 0:
        R = args.rotate
    else:
        R = int(min(8, max(1, math.ceil((1 << 30) / max(kv_bytes_touched, 1)))))
    caches = [(s.k_cache, s.v_cache)]
    for _ in range(R - 1):
        caches.append((s.k_cache.clone(), s.v_cache.clone()))
    slots = torch.empty(T, dtype=torch.int64, device=cuda)
    out = torch.empty((w.num_rows, w.q_len, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device=cuda)
    ws = K.make_workspace(w.num_rows, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim, cuda)
    stream = torch.cuda.current_stream(cuda)
    sp = int(stream.cuda_stream)
    dt = K.KVS_BF16 if w.dtype == "bf16" else K.KVS_F32
    flags = K.KVS_WALK_TABLE if table_walk else 0
    rows, stride = s.block_table.shape
    slot_args = (step_req.data_ptr(), step_pos.data_ptr(), T, T, s.block_table.data_ptr(),
                 int(rows), int(stride), w.block_size, slots.data_ptr(), sp)
    write_args = [(step_k.data_ptr(), step_v.data_ptr(), slots.data_ptr(), T, kc.data_ptr(),
                   vc.data_ptr(), w.total_blocks, w.block_size, w.num_kv_heads, w.head_dim, dt, sp)
                  for kc, vc in caches]
    if dcp:
        lse = torch.empty((w.num_rows, w.q_len, w.num_q_heads), dtype=torch.float32, device=cuda)
        f_attn = lib.paged_decode_attention_dcp
        attn_args = [(s.q.data_ptr(), kc.data_ptr(), vc.data_ptr(), s.block_table.data_ptr(),
                      int(stride), int(walk_blocks), s.seq_lens.data_ptr(), w.num_rows, w.q_len,
                      w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.total_blocks,
                      w.scale, dt, dcp[0], dcp[1], dcp[2], ws.data_ptr(), int(ws.numel()),
                      out.data_ptr(), lse.data_ptr(), sp) for kc, vc in caches]
    elif args.window:
        f_attn = lib.paged_decode_attention_swa
        wt = int(trimmed.shape[1])
        attn_args = [(s.q.data_ptr(), kc.data_ptr(), vc.data_ptr(), d_trim.data_ptr(), wt, wt,
                      s.seq_lens.data_ptr(), d_off.data_ptr(), int(args.window), w.num_rows, w.q_len,
                      w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.total_blocks,
                      w.scale, dt, ws.data_ptr(), int(ws.numel()), out.data_ptr(), sp)
                     for kc, vc in caches]
    else:
        f_attn = lib.paged_decode_attention
        attn_args = [(s.q.data_ptr(), kc.data_ptr(), vc.data_ptr(), s.block_table.data_ptr(),
                      int(stride), int(walk_blocks), s.seq_lens.data_ptr(), w.num_rows, w.q_len,
                      w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.total_blocks,
                      w.scale, dt, flags, ws.data_ptr(), int(ws.numel()), out.data_ptr(), sp)
                     for kc, vc in caches]
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # The default step is one paged_decode_attention_append call (the step's
    # write inside the decode launch when it qualifies); the sliding-window
    # and context-parallel steps have no append call.
    append = not (dcp or args.window or args.separate_write or args.fused_write)
    f_append = lib.paged_decode_attention_append
    append_args = [(step_req.data_ptr(), step_pos.data_ptr(), T, T, slots.data_ptr(),
                    step_k.data_ptr(), step_v.data_ptr(), s.q.data_ptr(), kc.data_ptr(),
                    vc.data_ptr(), s.block_table.data_ptr(), int(stride), int(walk_blocks),
                    s.seq_lens.data_ptr(), w.num_rows, w.q_len, w.num_q_heads, w.num_kv_heads,
                    w.head_dim, w.block_size, w.total_blocks, w.scale, dt, flags, ws.data_ptr(),
                    int(ws.numel()), out.data_ptr(), sp) for kc, vc in caches]
    f_slot, f_write = lib.kv_slot_mapping, lib.kv_cache_write
    f_fused = lib.kv_slot_mapping_cache_write
    f_slot_dcp = lib.kv_slot_mapping_dcp
    if dcp:
        slot_dcp_args = slot_args[:8] + tuple(dcp) + slot_args[8:]
    fused_args = [slot_args[:9] + (step_k.data_ptr(), step_v.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                   w.total_blocks, w.num_kv_heads, w.head_dim, dt, sp)
                  for kc, vc in caches]
    f_select = K.select_ctx_bucket

    def step(i, ev=None):
        # host: the per-step bucket pick the pages describe (feature off unless bucketed)
        f_select(max_ctx, num_spec, buckets, max_model_len, w.block_size)
        if batch_buckets:
            K.select_batch_bucket(num_active, batch_buckets)
        j = i % R
        if append:
            if ev is not None:
                ev[0].record(sp)
            st = f_append(*append_args[j])
            if ev is not None:
                ev[1].record(sp)
            if st:
                raise RuntimeError(f"library call failed with status {st}")
            return
        if dcp:
            st = f_slot_dcp(*slot_dcp_args)
            st |= f_write(*write_args[j])
        elif args.separate_write:
            st = f_slot(*slot_args)
            st |= f_write(*write_args[j])
        else:
            st = f_fused(*fused_args[j])
        if ev is not None:
            ev[0].record(sp)
        st |= f_attn(*attn_args[j])
        if ev is not None:
            ev[1].record(sp)
        if st:
            raise RuntimeError(f"library call failed with status {st}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: whole steps, back to back. The host stays ahead of the
    # GPU, so the wall time per step is GPU time.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # The step's attention call alone, each call bracketed by its own events
    # (a marker the GPU processes in line): median and mean of the durations.
    n_calls = max(args.calls, MIN_CALLS)
    events = [(HipEvent(), HipEvent()) for _ in range(n_calls)]
    for i, ev in enumerate(events):
        step(args.steps + i, ev)
    torch.cuda.synchronize()
    durations = np.array([e0.elapsed_ms(e1) for e0, e1 in events]) * 1e-3
    t_attn = float(np.median(durations))
    t_attn_mean = float(np.mean(durations))

    # Slot mapping and cache write on their own: back-to-back launches
    # between two events give each kernel's time in a busy stream.
    def back_to_back(fn, arg_list, n):
        e0, e1 = HipEvent(), HipEvent()
        for k in range(min(n, 10)):
            fn(*arg_list[k % len(arg_list)])
        e0.record(sp)
        for k in range(n):
            if fn(*arg_list[k % len(arg_list)]):
                raise RuntimeError("library call failed")
        e1.record(sp)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) * 1e-3 / n

    t_slot = back_to_back(f_slot, [slot_args], args.steps)
    t_write = back_to_back(f_write, write_args, args.steps)
    t_fused = back_to_back(f_fused, fused_args, args.steps)
    # With the append step, the attention call on its own (back to back, the
    # caches already holding the step's rows) for reference.
    t_attn_only = back_to_back(f_attn, attn_args, args.steps) if append else t_attn

    # Under context parallelism the ranks' (out, lse) would be all-gathered
    # and merged by decode_lse_merge; one GPU holds only rank 0's share, so
    # the merge is timed on world copies of it (its cost depends on the
    # shapes, not the values).
    lse_merge = None
    if dcp:
        world = dcp[0]
        rows_m = w.num_rows * w.q_len * w.num_q_heads
        outs = out.reshape(1, rows_m, w.head_dim).expand(world, -1, -1).contiguous()
        lses = lse.reshape(1, rows_m).expand(world, -1).contiguous()
        m_out = torch.empty((rows_m, w.head_dim), dtype=torch.float32, device=cuda)
        m_lse = torch.empty(rows_m, dtype=torch.float32, device=cuda)
        m_args = (outs.data_ptr(), lses.data_ptr(), world, rows_m, w.head_dim, m_out.data_ptr(),
                  m_lse.data_ptr(), sp)
        t_m = back_to_back(lib.decode_lse_merge, [m_args], 100)
        m_bytes = (world + 1) * rows_m * (w.head_dim + 1) * 4
        lse_merge = {"world": world, "rows": rows_m, "us": round(t_m * 1e6, 3),
                     "algorithmic_bytes": m_bytes, "gbps": round(m_bytes / t_m / 1e9, 2)}

    # Slot mapping at 2^22 tokens per launch (the step's few tokens only
    # measure the launch): tokens of random real requests at random positions
    # below their context lengths, mapped through this workload's table. The
    # launches rotate over SLOT_SWEEP_SETS distinct token sets (about 1.1 GB of
    # token and slot arrays), so their bytes come from HBM and not from the
    # 256 MB last-level cache; only the table (a few hundred KB) stays cached.
    sweep = sweep_chunked = None
    if w.num_reqs:
        nt = SLOT_SWEEP_TOKENS
        gen = torch.Generator(device=cuda)
        gen.manual_seed(w.seed + 7)
        lens = torch.from_numpy(np.maximum(w.seq_lens[: w.num_reqs].astype(np.int64), 1)).to(cuda)
        sets = []
        for _ in range(SLOT_SWEEP_SETS):
            d_req = torch.randint(0, w.num_reqs, (nt,), generator=gen, device=cuda,
                                  dtype=torch.int64)
            d_pos = (torch.rand(nt, generator=gen, device=cuda, dtype=torch.float64)
                     * lens[d_req]).to(torch.int64)
            d_req = d_req.to(torch.int32)
            d_slots = torch.empty(nt, dtype=torch.int64, device=cuda)
            sets.append((d_req, d_pos, d_slots))
        big = [(a.data_ptr(), b.data_ptr(), nt, nt, s.block_table.data_ptr(), int(rows),
                int(stride), w.block_size, c.data_ptr(), sp) for a, b, c in sets]
        t_big = back_to_back(f_slot, big, 5 * SLOT_SWEEP_SETS)
        sweep = {"tokens": nt, "token_sets_rotated": SLOT_SWEEP_SETS,
                 "distinct_bytes": slot_map_bytes(nt) * SLOT_SWEEP_SETS,
                 "us": round(t_big * 1e6, 3),
                 "tokens_per_s": round(nt / t_big, 1),
                 "gbps": round(slot_map_bytes(nt) / t_big / 1e9, 2),
                 "frac_of_peak": round(slot_map_bytes(nt) / t_big / 1e9 / HBM_PEAK_GBPS, 4),
                 "note": "24 B per token counted; requests and positions drawn at random, so "
                         "every table read is a scattered cache-line fetch (the worst case; a "
                         "step's tokens are grouped by request); the token and slot arrays "
                         "stream from HBM"}
        del sets
        # The same sweep with the tokens of a prefill chunk: runs of
        # SLOT_SWEEP_RUN consecutive positions of one request (a random real
        # request, from a random start below its length), as a chunked step
        # hands them over; neighbouring tokens then share their table entry.
        runs = nt // SLOT_SWEEP_RUN
        step = torch.arange(SLOT_SWEEP_RUN, device=cuda, dtype=torch.int64)
        sets = []
        for _ in range(SLOT_SWEEP_SETS):
            r_req = torch.randint(0, w.num_reqs, (runs,), generator=gen, device=cuda,
                                  dtype=torch.int64)
            r_len = lens[r_req]
            r_start = (torch.rand(runs, generator=gen, device=cuda, dtype=torch.float64)
                       * torch.clamp(r_len - SLOT_SWEEP_RUN, min=1)).to(torch.int64)
            d_pos = torch.minimum(r_start[:, None] + step[None, :], r_len[:, None] - 1).reshape(-1)
            d_req = r_req.to(torch.int32).repeat_interleave(SLOT_SWEEP_RUN)
            d_slots = torch.empty(nt, dtype=torch.int64, device=cuda)
            sets.append((d_req.contiguous(), d_pos.contiguous(), d_slots))
        big = [(a.data_ptr(), b.data_ptr(), nt, nt, s.block_table.data_ptr(), int(rows),
                int(stride), w.block_size, c.data_ptr(), sp) for a, b, c in sets]
        t_chunk = back_to_back(f_slot, big, 5 * SLOT_SWEEP_SETS)
        sweep_chunked = {"tokens": nt, "token_sets_rotated": SLOT_SWEEP_SETS,
                         "run": SLOT_SWEEP_RUN, "us": round(t_chunk * 1e6, 3),
                         "tokens_per_s": round(nt / t_chunk, 1),
                         "gbps": round(slot_map_bytes(nt) / t_chunk / 1e9, 2),
                         "frac_of_peak": round(slot_map_bytes(nt) / t_chunk / 1e9 / HBM_PEAK_GBPS, 4),
                         "note": f"24 B per token counted; runs of {SLOT_SWEEP_RUN} consecutive "
                                 "positions of one request (a prefill chunk), so neighbouring "
                                 "tokens share their table entry; the token and slot arrays "
                                 "stream from HBM"}
        del sets

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=cuda).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    write_bytes = cache_write_bytes(w, T_live, T)
    if not (args.separate_write or dcp):
        write_bytes -= 8 * T  # the one-launch write keeps the slots in registers
    step_bytes = slot_map_bytes(T) + write_bytes + a_bytes
    decode_tokens = w.num_reqs * w.q_len
    attn_gbps = a_bytes / t_attn_only / 1e9
    # the call the timed steps make: with the append it also moves the step's
    # slots and rows, and is credited with those bytes
    call_bytes = step_bytes if append else a_bytes
    call_gbps = call_bytes / t_attn / 1e9
    result = {
        "metric": "paged decode attention HBM GB/s (% of peak) + decode tokens/s; slot_map tok/s",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded block permutation; no dataset)",
        "config": {
            "workload": (DESCRIPTIONS["3spec"].format(n=args.num_spec) if args.num_spec
                         else DESCRIPTIONS[idx]),
            "seed": w.seed,
            "max_ctx": int((w.computed + w.chunk_lens)[: w.num_reqs].max()),
            "num_seqs": w.num_rows,
            "batch_buckets": batch_buckets,
            "q_len": w.q_len,
            "walk": f"window {args.window} (tail-trimmed table)" if args.window else args.walk,
            "walk_blocks": int(walk_blocks),
            "bucket_len": int(bucket_len),
            "step_tokens": T,
            "cache_copies_rotated": R,
            "step_write": ("in the decode call (paged_decode_attention_append)" if append else
                           "separate" if (args.separate_write or dcp) else "fused"),
            "dcp": {"world": dcp[0], "rank": dcp[1], "interleave": dcp[2]} if dcp else None,
            "tp": args.tp,
            "heads": {"kv": w.num_kv_heads, "q": w.num_q_heads},
            "parallelism": ("single GPU" if args.tp == 1 else
                            f"single GPU: one rank's share under tensor parallelism {args.tp}"),
        },
        "attention_gbps": round(attn_gbps, 2),
        "attention_frac_of_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "attention_gbps_token_exact": (round(exact_bytes / t_attn_only / 1e9, 2)
                                       if exact_bytes is not None else None),
        "decode_tokens_per_s": round(decode_tokens / (ms_per_step * 1e-3), 1),
        "slot_map_tokens_per_s": round(T / t_slot, 1),
        "slot_map_sweep": sweep,
        "slot_map_sweep_chunked": sweep_chunked,
        "lse_merge": lse_merge,
        "kernel_us": {"kv_slot_mapping": round(t_slot * 1e6, 3),
                      "kv_cache_write": round(t_write * 1e6, 3),
                      "kv_slot_mapping_cache_write": round(t_fused * 1e6, 3),
                      "paged_decode_attention": round(t_attn_only * 1e6, 3),
                      "paged_decode_attention_append": round(t_attn * 1e6, 3) if append else None},
        "algorithmic_bytes": {"kv_slot_mapping": slot_map_bytes(T),
                              "kv_cache_write": cache_write_bytes(w, T_live, T),
                              "paged_decode_attention": a_bytes,
                              "paged_decode_attention_token_exact": exact_bytes,
                              "paged_decode_attention_append": call_bytes if append else None},
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_decode_attention_append (the step's slots and rows written "
                       "inside; their bytes credited)" if append else "paged_decode_attention"),
            "achieved": round(call_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(call_gbps / HBM_PEAK_GBPS, 4),
            "calls": n_calls,
            "call_us_median": round(t_attn * 1e6, 3),
            "call_us_mean": round(t_attn_mean * 1e6, 3),
            "call_us_p10_p90": [round(float(np.percentile(durations, 10)) * 1e6, 3),
                                round(float(np.percentile(durations, 90)) * 1e6, 3)],
            "traffic": measured_traffic(args.workload, variant_key(args)),
        },
        "setup_s": round(t_setup, 2),
    }
    # bytes of the attention launches of this walk: what the method needs
    # (algorithmic, whole blocks) and what the counters measured (DRAM)
    result["walk_bytes"] = {"walk": result["config"]["walk"], "algorithmic": a_bytes,
                            "measured_dram": result["roofline"]["traffic"]}
    if not args.no_cpu_baseline and not dcp:
        result["cpu_baseline"] = cpu_baseline(w, s.host_table, walk_blocks, args.cpu_seconds,
                                              window=args.window)
    print(json.dumps(result), flush=True)
    return 0


def variant_key(args) -> str:
    """Name of the measured variant of a workload, as the counter summaries
    under profiles/ are keyed: the walk, or the sliding window, the
    context-parallel or tensor-parallel share, the speculative tokens, and a
    forced largest context."""
    if args.window:
        key = f"window{args.window}"
    elif args.dcp > 1:
        key = f"dcp{args.dcp}"
    elif args.tp > 1:
        key = f"tp{args.tp}"
    elif args.num_spec:
        key = f"spec{args.num_spec}"
    else:
        key = args.walk
    if args.max_ctx is not None:
        key += f"_maxctx{args.max_ctx}"
    return key


def measured_traffic(workload: str, walk: str):
    """HBM bytes per launch from the committed counter summary, or None.

    The summary records the hash of the kernel code it was taken with
    (kernel_source_hash); once the code has changed the figure no longer
    applies and None is reported.
    """
    path = os.path.join(ROOT, "profiles", f"paged_decode_attention_{workload}_{walk}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def host_cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """CPU threads this process may use: its affinity set, capped by
    OMP_NUM_THREADS when that is set (the share of a host the GPU job has)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(n, 1)


def cpu_baseline(w, table, walk_blocks, seconds, window=0, sample_reqs=16):
    """The oracle as it stands, on the host cores, over a bounded sample.

    Untimed: the oracle builds its own caches (prefill + step writes) for a
    sample of the batch's requests (the first ``sample_reqs`` real ones).
    Timed, twice: the oracle's paged_decode_attention, one request per call,
    cycling over the sample until ``seconds`` have passed; first on one
    thread, then on a pool of host_threads() threads, each call one request
    (numpy's BLAS calls and large copies release the GIL). BLAS is pinned to
    one thread per caller in both legs. Throughput is the algorithmic
    attention bytes of the requests processed per second.
    """
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle.runner import OracleStep

    real = [i for i in range(w.num_reqs) if w.seq_lens[i] > 0][:sample_reqs]
    es = w.es
    per_block = 2 * w.block_size * w.num_kv_heads * w.head_dim * es + 4
    per_req_fixed = w.q_len * w.num_q_heads * w.head_dim * (es + 4) + 4

    def req_bytes(rr):
        L = int(w.seq_lens[rr])
        vis = min(L, walk_blocks * w.block_size)
        first = max(0, L - w.q_len - window + 1) // w.block_size if window else 0
        return (-(-vis // w.block_size) - first) * per_block + per_req_fixed

    with threadpool_limits(limits=1):
        ref = OracleStep(w, table, requests=real, full_image=False)
        ref.write_step()
        q = w.q()

        def one(rr):
            ref.attention(q, walk_blocks=walk_blocks, requests=[rr], window=window)
            return req_bytes(rr)

        legs = {}
        for threads in (1, host_threads()):
            done_bytes, n, r = 0, 0, 0
            t0 = time.perf_counter()
            if threads == 1:
                while time.perf_counter() - t0 < seconds:
                    done_bytes += one(real[r % len(real)])
                    n += 1
                    r += 1
            else:
                with ThreadPoolExecutor(max_workers=threads) as pool:
                    while time.perf_counter() - t0 < seconds:
                        batch = [real[(r + i) % len(real)] for i in range(threads)]
                        done_bytes += sum(pool.map(one, batch))
                        n += threads
                        r += threads
            el = time.perf_counter() - t0
            legs[threads] = (done_bytes / el / 1e9, n, el)
    model = host_cpu_model()
    nthr = max(legs)
    gbps, n, el = legs[nthr]
    g1, n1, el1 = legs[1]
    return {
        "value": round(gbps, 6),
        "unit": "GB/s",
        "cores": nthr,
        "kind": "oracle",
        "sample": f"oracle fp64 paged_decode_attention over {len(real)} requests of this "
                  f"workload, one request per call, cycled: {n} calls in {el:.1f} s on {nthr} "
                  f"threads (BLAS 1 thread each); host {model}, {os.cpu_count()} logical CPUs, "
                  f"{len(os.sched_getaffinity(0))} in this process's affinity set",
        "cpu_model": model,
        "single_core": {"value": round(g1, 6), "unit": "GB/s", "cores": 1,
                        "sample": f"{n1} calls in {el1:.1f} s on one thread"},
    }


if __name__ == "__main__":
    sys.exit(main())
